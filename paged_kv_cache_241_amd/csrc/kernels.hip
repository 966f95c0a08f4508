// HIP kernels for gfx950 (CDNA4): KV append, copy-on-write block copies and
// single-token decode attention over a paged (or per-request contiguous)
// KV cache.
//
// What is computed follows the pages:
//   * append: each decode iteration adds one token per request ("Insights into
//     LLM Serving Systems: KV-Cache Memory Allocation Patterns", section 4,
//     Observation-1); its K and V rows are bit-copied into the slot the host
//     allocator gave it;
//   * copy_blocks: a shared block is copied when a sharer first writes into it
//     (PagedAttention summary page, Summary; "Running Out of Cache",
//     "Fragmentation is lost users");
//   * decode: attention of one query token per request over K/V held in fixed
//     blocks reached through a block table ("Running Out of Cache", paging
//     paragraph and Terms), or over a per-request sub-tensor at reqId x S
//     ("Leveraging Low-Level CUDA APIs for vAttention's Dynamic Memory",
//     5.2.3).
//
// Decode design (the pages give no kernel; this one is built for gfx950):
//   * one 256-thread workgroup (4 waves of 64) per (sequence, KV head, context
//     partition); the G <= 16 query heads of the GQA group share every K/V
//     load; waves take the partition's 16-token chunks round-robin from its
//     end, so that the context's last chunk (the one that may be partly
//     filled, and the one the fused append patches) is a wave's first;
//   * per chunk, S = K q^T is one 16x16 MFMA tile (16 tokens x 16 head
//     columns, the unused columns hold zero queries): bf16 caches use
//     v_mfma_f32_16x16x32_bf16 over head_dim/32 steps, fp32 caches
//     v_mfma_f32_16x16x4_f32 over head_dim/4 steps.  The lane that holds
//     S[token 4j+i][head n] is exactly the lane the P V MFMA wants P[head n]
//     [token 4j+i] in, so the softmax weights never move between lanes;
//   * online softmax in fp32 (exp2 on pre-scaled scores), one running max per
//     head; P V: bf16 caches split each weight into a bf16 high and low part
//     (two v_mfma_f32_16x16x16_bf16 per 16x16 output tile, weights exact to
//     ~2^-17), fp32 caches multiply fp32 weights with v_mfma_f32_16x16x4_f32;
//   * the tile formats make every operand load one contiguous wave access:
//     K chunks [D/VE][BS][VE] give 1 KiB per load, V [D][BS] 512 B (bf16);
//   * waves merge through LDS in a fixed order; partitions are merged by a
//     second small kernel in partition order.  Every reduction order depends
//     only on logical token positions, so results do not depend on which
//     physical blocks hold the tokens, nor on paged vs contiguous storage;
//   * grids of at most one wave per SIMD (a batch of one or two long
//     contexts) keep two chunks' loads in flight per wave (two operand sets
//     in registers); grids of at most two waves per SIMD let the waves that
//     hold one chunk more than the others load their first two chunks
//     together; fuller grids hide the HBM latency with resident waves;
//   * a launch split into partitions runs from a work plan (one small
//     kernel): only partitions holding tokens, full ones first and each
//     context's last one longest first, so that the grid holds no empty
//     workgroups among the others and ends on short ones.
// The partition kernel's body is in decode_partition.hpp (the shared-prefix
// launch runs it too).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "decode_common.hpp"
#include "decode_partition.hpp"
#include "kernels.hpp"

// Split-K partials and the work plan of pa_append_decode_noalloc, for callers
// that cannot allocate.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address static_scratch() looks up is passed on.
static __device__ __align__(256) unsigned char scratch[pa::kStaticScratchBytes];

namespace pa {
namespace {

constexpr int kMergeWaves = 4;   // merge rows per workgroup, one a wave
constexpr int kMergeUnroll = 8;  // rows of up to this many partitions load all at once (at most)
constexpr int kMaxGroup = 16;     // query heads per KV head the tile can hold

template <int KIND, int D, int BS, int W, bool NT, bool PIPE, bool BAL = false>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<KIND, BS, PIPE, BAL>())))
void decode_partition_kernel(CacheGeom geo, DecodeArgs a) {
  extern __shared__ float lds[];
  decode_partition_body<KIND, D, BS, W, NT, PIPE, BAL>(geo, a, blockIdx.x, gridDim.x, lds);
}

// Work plan of a launch split into partitions: plan[i] = {s * P + part, L_s}
// for the i-th (sequence, partition) with tokens to attend, {-1, 0} past the
// last.  Full partitions come first (in sequence order for up to 1024
// sequences), then every context's last partition, longest first
// (kPlanBuckets length classes; the order within a class varies between
// runs, which changes no result: each partition is computed on its own and
// merged in partition order).  Shared prefixes (seq_shared) are left out.
// The partition kernel's grid then ends
// on its shortest workgroups, and the items without work (contexts shorter
// than the longest) come after all others instead of among them.  One
// workgroup.
constexpr int kPlanThreads = 1024;
constexpr int64_t kPlanMinGrid = 2048;  // two rounds of resident workgroups (256 CUs x 4)
constexpr int kPlanBuckets = 64;  // one per lane of a wave
constexpr int kPlanKeep = 4;      // sequences per thread kept in registers

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a, int2* __restrict__ plan) {
  static_assert(kPlanBuckets == kWave, "one length class per lane");
  __shared__ int hist[kPlanBuckets];
  __shared__ int cursor[kPlanBuckets];
  __shared__ int wsum[kPlanThreads / kWave];
  __shared__ int total;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int B = a.num_seqs, P = a.num_partitions, pc = a.partition_chunks;
  // sequence s: L, partitions [first, np) hold its unshared tokens, the last
  // one has `last` chunks
  struct Span { int L, first, np, last; };
  auto span = [&](int s) -> Span {
    Span r;
    r.L = a.lens[s];
    const int nch = (r.L + kChunk - 1) / kChunk;
    r.np = min((nch + pc - 1) / pc, P);
    r.first = a.seq_shared != nullptr ? min(a.seq_shared[s] / (pc * kChunk), r.np) : 0;
    r.last = r.np > 0 ? min(nch - (r.np - 1) * pc, pc) : 0;
    return r;
  };
  // length class, 0 for the longest last partitions
  auto bucket = [&](int last) { return kPlanBuckets - 1 - ((last - 1) * kPlanBuckets) / pc; };
  if (tid < kPlanBuckets) hist[tid] = 0;
  Span keep[kPlanKeep];
#pragma unroll
  for (int k = 0; k < kPlanKeep; ++k)
    keep[k] = tid + k * kPlanThreads < B ? span(tid + k * kPlanThreads) : Span{0, 0, 0, 0};
  __syncthreads();
  int mine = 0;  // full partitions of this thread's sequences
  auto count = [&](const Span& r) {
    if (r.np > r.first) {
      mine += r.np - 1 - r.first;
      atomicAdd(&hist[bucket(r.last)], 1);
    }
  };
#pragma unroll
  for (int k = 0; k < kPlanKeep; ++k) count(keep[k]);
  for (int s = tid + kPlanKeep * kPlanThreads; s < B; s += kPlanThreads) count(span(s));
  const int x = wave_incl_scan(mine, lane);
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    // offsets of the waves' full partitions, then of the length classes
    // after all full partitions, longest class first
    const int v = wave_incl_scan(lane < kPlanThreads / kWave ? wsum[lane] : 0, lane);
    if (lane < kPlanThreads / kWave) wsum[lane] = v;
    const int full = __shfl(v, kPlanThreads / kWave - 1);
    const int h = hist[lane];
    const int hs = wave_incl_scan(h, lane);
    cursor[lane] = full + hs - h;
    if (lane == kWave - 1) total = full + hs;
  }
  __syncthreads();
  int pos = (wave > 0 ? wsum[wave - 1] : 0) + x - mine;
  auto place = [&](int s, const Span& r) {
    for (int p = r.first; p < r.np - 1; ++p) plan[pos++] = make_int2(s * P + p, r.L);
    if (r.np > r.first) plan[atomicAdd(&cursor[bucket(r.last)], 1)] = make_int2(s * P + r.np - 1, r.L);
  };
#pragma unroll
  for (int k = 0; k < kPlanKeep; ++k)
    if (tid + k * kPlanThreads < B) place(tid + k * kPlanThreads, keep[k]);
  for (int s = tid + kPlanKeep * kPlanThreads; s < B; s += kPlanThreads) place(s, span(s));
  for (int i = total + tid; i < B * P; i += kPlanThreads) plan[i] = make_int2(-1, 0);
}

// Merge context partitions in partition order: one wave per (seq, q head),
// kMergeWaves rows per workgroup, D / 64 output dims a lane.  Rows of up to
// U partitions (2, 4 or kMergeUnroll: the launch's partition count rounded
// up) issue all their loads (maxima and sums as scalar loads, partial
// outputs as vector loads) before any arithmetic; longer rows find their
// maximum 64 partitions a round in the lanes, then load and sum U partitions
// at a time.  The sums run over p in order, as fma(w_p, acc_p, .) and
// fma(w_p, l_p, .), whatever U is.
template <int D, int U>
__global__ __launch_bounds__(kMergeWaves * kWave) void decode_merge_kernel(DecodeArgs a) {
  constexpr int E = D / kWave;
  static_assert(E * kWave == D, "D is a multiple of the wave");
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * kMergeWaves +
                     __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (sh >= rows) return;
  const int s = static_cast<int>(sh / a.num_q_heads);
  const int P = a.num_partitions;
  const int L = a.lens[s];
  const int tp = a.partition_chunks * kChunk;
  const int ps = min((L + tp - 1) / tp, P);
  const float* ml = a.ws + sh * P * 2;
  const float* accp = a.ws + rows * P * 2 + sh * P * D + lane * E;
  float* o = a.out + sh * D + lane * E;
  float A[E];
#pragma unroll
  for (int e = 0; e < E; ++e) A[e] = 0.0f;
  if (ps > 0 && ps <= U) {
    // all of the row's loads at once (indices clamped into [0, ps), the
    // copies past ps weigh nothing), then the same sums as below
    float mp[U], lp[U], ap[U][E];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int p = min(k, ps - 1);
      mp[k] = ml[2 * p];
      lp[k] = ml[2 * p + 1];
#pragma unroll
      for (int e = 0; e < E; ++e) ap[k][e] = accp[p * D + e];
    }
    // (the clamped copies repeat partition ps - 1: the max is unchanged)
    float mx = mp[0];
#pragma unroll
    for (int k = 1; k < U; ++k) mx = fmaxf(mx, mp[k]);
    // selects rather than branches, so that every load is used and issued
    // up front
    float Lt = 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float wt = fexp2(mp[k] - mx);
      const bool live = k < ps;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float t = fmaf(wt, ap[k][e], A[e]);
        A[e] = live ? t : A[e];
      }
      const float lt = fmaf(wt, lp[k], Lt);
      Lt = live ? lt : Lt;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) A[e] = A[e] / Lt;
  } else if (ps > 0) {
    // the maximum over all partitions (64 a round in the lanes), then the
    // sums in groups of U partitions whose loads issue together
    float mx = -INFINITY;
    for (int p0 = 0; p0 < ps; p0 += kWave)
      if (p0 + lane < ps) mx = fmaxf(mx, ml[2 * (p0 + lane)]);
#pragma unroll
    for (int x = kWave / 2; x >= 1; x /= 2) mx = fmaxf(mx, __shfl_xor(mx, x));
    float Lt = 0.0f;
    for (int p0 = 0; p0 < ps; p0 += U) {
      float mp[U], lp[U], ap[U][E];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int p = min(p0 + k, ps - 1);
        mp[k] = ml[2 * p];
        lp[k] = ml[2 * p + 1];
#pragma unroll
        for (int e = 0; e < E; ++e) ap[k][e] = accp[static_cast<int64_t>(p) * D + e];
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const float wt = fexp2(mp[k] - mx);
        const bool live = p0 + k < ps;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float t = fmaf(wt, ap[k][e], A[e]);
          A[e] = live ? t : A[e];
        }
        const float lt = fmaf(wt, lp[k], Lt);
        Lt = live ? lt : Lt;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) A[e] = A[e] / Lt;
  }
  // the output is not read again here: non-temporal stores (0.1-0.4% on
  // the ragged mix, the shared-prefix step and batches of 1-4 long contexts)
  if constexpr (E == 2) {
    typedef float floatx2_t __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(floatx2_t{A[0], A[1]}, reinterpret_cast<floatx2_t*>(o));
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) __builtin_nontemporal_store(A[e], &o[e]);
  }
}

// ---------------------------------------------------------------------------
// append and copy-on-write copies
// ---------------------------------------------------------------------------
// One (token, KV head, 16-byte piece of the row) of an append: the K piece
// is stored whole, the V piece's elements go to their dims' rows of the V
// tile.  idx = (token * num_kv_heads + head) * pieces + piece.
__device__ __forceinline__ void append_item(const CacheGeom& g, int32_t layer, const uint4* __restrict__ k,
                                            const uint4* __restrict__ v, const int32_t* __restrict__ slots,
                                            int64_t idx) {
  const int ve = 16 / g.elt;
  const int chunks = g.head_dim / ve;
  const int per_tok = g.num_kv_heads * chunks;
  const int i = static_cast<int>(idx / per_tok);
  const int rem = static_cast<int>(idx % per_tok);
  const int h = rem / chunks, q = rem % chunks;
  const int slot = slots[i];
  if (slot < 0) return;
  const int64_t u = slot / g.block_size;
  // the row's tile pair in its (block, head): pairs of up to 16 rows
  const int sub = g.block_size < 16 ? g.block_size : 16;
  const int o = slot % g.block_size % sub;
  const int64_t sub_bytes = static_cast<int64_t>(g.head_dim) * sub * g.elt;
  char* kt = g.base + static_cast<int64_t>(layer) * g.layer_bytes + (u * g.num_kv_heads + h) * 2 * g.tile_bytes +
             (slot % g.block_size / sub) * 2 * sub_bytes;
  *reinterpret_cast<uint4*>(kt + (static_cast<int64_t>(q) * sub + o) * 16) = k[idx];
  const uint4 w = v[idx];
  char* vt = kt + sub_bytes;
  const int d0 = q * ve;
  if (g.elt == 2) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint16_t*>(vt + ((d0 + 2 * e) * sub + o) * 2) = static_cast<uint16_t>(ws[e] & 0xFFFFu);
      *reinterpret_cast<uint16_t*>(vt + ((d0 + 2 * e + 1) * sub + o) * 2) = static_cast<uint16_t>(ws[e] >> 16);
    }
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint32_t*>(vt + ((d0 + e) * sub + o) * 4) = ws[e];
  }
}

// One thread per (token, KV head, 16-byte piece of the row): the decode
// step's append (one scattered token per sequence).
__global__ __launch_bounds__(256) void append_kv_kernel(CacheGeom g, int32_t layer,
                                                        const uint4* __restrict__ k,
                                                        const uint4* __restrict__ v,
                                                        const int32_t* __restrict__ slots,
                                                        int32_t n) {
  const int64_t per_tok = static_cast<int64_t>(g.num_kv_heads) * (g.head_dim * g.elt / 16);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * per_tok) return;
  append_item(g, layer, k, v, slots, idx);
}

// Appends of many tokens (prompt ingestion): the same items as
// append_kv_kernel, in windows of 16 tokens ordered token-fastest, so that
// 16 lanes of a wave hold consecutive tokens of one (head, piece).  A
// prefill's consecutive tokens sit in consecutive rows of a block's tiles:
// those lanes' K pieces then form one 256-byte run and their V elements
// whole 32-byte rows, which the memory system merges into full-sector writes
// instead of 2-byte ones; each lane group reads 64 contiguous bytes a token.
constexpr int kBulkMinTokens = 256;   // appends of fewer tokens use append_kv_kernel

__global__ __launch_bounds__(256) void append_kv_bulk_kernel(CacheGeom g, int32_t layer,
                                                             const uint4* __restrict__ k,
                                                             const uint4* __restrict__ v,
                                                             const int32_t* __restrict__ slots,
                                                             int32_t n) {
  const int64_t pieces = static_cast<int64_t>(g.num_kv_heads) * (g.head_dim * g.elt / 16);
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  // windows of 16 tokens: token-fastest inside a window, then (head, piece)
  const int64_t win = x / (16 * pieces), r = x % (16 * pieces);
  const int64_t token = win * 16 + r % 16, hp = r / 16;  // hp: head * pieces-per-head + piece
  if (token >= n) return;
  append_item(g, layer, k, v, slots, token * pieces + hp);
}

// Workgroup (pair, layer) copies block src's tile pairs of the layer (every
// KV head, K and V: one contiguous run) onto block dst's.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CacheGeom g,
                                                          const int32_t* __restrict__ pairs) {
  const int pi = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
  const int64_t bb = static_cast<int64_t>(g.num_kv_heads) * 2 * g.tile_bytes;
  const int64_t lb = static_cast<int64_t>(layer) * g.layer_bytes;
  const uint4* s = reinterpret_cast<const uint4*>(g.base + lb + src * bb);
  uint4* d = reinterpret_cast<uint4*>(g.base + lb + dst * bb);
  for (int64_t x = threadIdx.x; x < bb / 16; x += 256) d[x] = s[x];
}

template <int KIND, int D, int BS, bool PIPE, bool BAL = false>
hipError_t launch_decode_p(const CacheGeom& g, const DecodeArgs& a, hipStream_t st) {
  constexpr int W = kDecodeWaves;
  const int64_t nwork = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
  const int G = a.num_q_heads / g.num_kv_heads;
  const size_t lds = static_cast<size_t>(merge_lds_bytes(W, G, D)) +
                     (a.new_k != nullptr ? append_lds_bytes(D, g.elt, BS) : 0);
  if (a.streaming)
    hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, W, true, PIPE, BAL>), dim3(static_cast<uint32_t>(nwork)),
                       dim3(W * kWave), lds, st, g, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, W, false, PIPE, BAL>), dim3(static_cast<uint32_t>(nwork)),
                       dim3(W * kWave), lds, st, g, a);
  return hipGetLastError();
}

// Grids of at most kPipeMaxWaves waves (one per SIMD: a batch of one or two
// long contexts) run the two-chunk pipeline: with one chunk in flight per
// wave they wait out an HBM round trip per chunk.  Measured on MI355X,
// Llama-3-8B shape: batch 1 x 8192 tokens 15.1 -> 13.5 us, batch 1 x 2048
// 12.2 -> 10.3 us.  Fuller grids keep one chunk in flight (at two waves per
// SIMD the pipeline gained 1-2% at batch 4-8 and lost 1.6% on the Yi-34B
// share).
constexpr int64_t kPipeMaxWaves = 1024;
// Grids of at most two waves per SIMD (e.g. 64 sequences x 8 KV heads, one
// partition each) run the balanced start: its first step holds a second
// operand set (141 VGPRs, three waves per SIMD, more than such a grid
// places), which four waves per SIMD could not afford.
constexpr int64_t kBalancedMaxWaves = 2048;

template <int KIND, int D, int BS>
hipError_t launch_decode_t(const CacheGeom& g, const DecodeArgs& a, hipStream_t st) {
  if constexpr (decode_pipe_ok<KIND, BS>()) {
    const int64_t nwork = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
    if (a.plan == nullptr && nwork * kDecodeWaves <= kPipeMaxWaves) return launch_decode_p<KIND, D, BS, true>(g, a, st);
    if (a.plan == nullptr && nwork * kDecodeWaves <= kBalancedMaxWaves)
      return launch_decode_p<KIND, D, BS, false, true>(g, a, st);
  }
  return launch_decode_p<KIND, D, BS, false>(g, a, st);
}

template <int D>
hipError_t launch_merge_d(const DecodeArgs& a, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  // rows load all their partitions at once up to U: the fewest loads that
  // still cover the launch's partition count (clamped copies weigh nothing)
  const dim3 grid(static_cast<uint32_t>((rows + kMergeWaves - 1) / kMergeWaves)), block(kMergeWaves * kWave);
  if (a.num_partitions <= 2) hipLaunchKernelGGL((decode_merge_kernel<D, 2>), grid, block, 0, st, a);
  else if (a.num_partitions <= 4) hipLaunchKernelGGL((decode_merge_kernel<D, 4>), grid, block, 0, st, a);
  else if (a.num_partitions <= 8) hipLaunchKernelGGL((decode_merge_kernel<D, 8>), grid, block, 0, st, a);
  else if (a.num_partitions <= 16) hipLaunchKernelGGL((decode_merge_kernel<D, 16>), grid, block, 0, st, a);
  else if (a.num_partitions <= 32) hipLaunchKernelGGL((decode_merge_kernel<D, 32>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((decode_merge_kernel<D, kMergeUnroll>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int KIND, int D>
hipError_t launch_decode_bs(const CacheGeom& g, const DecodeArgs& a, bool* ok, hipStream_t st) {
  switch (g.block_size) {
    case 8: return launch_decode_t<KIND, D, 8>(g, a, st);
    case 16: return launch_decode_t<KIND, D, 16>(g, a, st);
    case 32: return launch_decode_t<KIND, D, 32>(g, a, st);
    default: *ok = false; return hipSuccess;
  }
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  // one lookup per device, with that device current; each GPU holds its own
  // copy of the array at its own address
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_append(const CacheGeom& g, int32_t layer, const void* k, const void* v,
                         const int32_t* slots, int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = static_cast<int64_t>(n) * g.num_kv_heads * (g.head_dim * g.elt / 16);
  const uint32_t blocks = static_cast<uint32_t>((threads + 255) / 256);
  if (n >= kBulkMinTokens) {
    // whole 16-token windows (the last one partly empty)
    const int64_t wthreads = static_cast<int64_t>((n + 15) / 16) * 16 * g.num_kv_heads * (g.head_dim * g.elt / 16);
    const uint32_t wblocks = static_cast<uint32_t>((wthreads + 255) / 256);
    hipLaunchKernelGGL(append_kv_bulk_kernel, dim3(wblocks), dim3(256), 0, stream, g, layer,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots, n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(append_kv_kernel, dim3(blocks), dim3(256), 0, stream, g, layer,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots, n);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CacheGeom& g, const int32_t* pairs, int32_t n,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(n), g.num_layers), dim3(256),
                     0, stream, g, pairs);
  return hipGetLastError();
}

hipError_t launch_merge(const CacheGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs <= 0 || a.num_partitions <= 1) return hipSuccess;
  return g.head_dim == 128 ? launch_merge_d<128>(a, stream) : launch_merge_d<64>(a, stream);
}

namespace {
int2* plan_place(const CacheGeom& g, const DecodeArgs& a) {
  // the plan follows the partials in the workspace
  return reinterpret_cast<int2*>(a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads *
                                            a.num_partitions * (g.head_dim + 2));
}
}  // namespace

// Large split launches run from a plan (decode_plan_kernel).  Below
// kPlanMinGrid workgroups the plan's launch (~3 us) costs more than it saves
// (measured: batch 1-16 with contexts of 4-8 K tokens); after a shared-prefix
// pass every context has one private partition left, and the plan does not
// pay either.
bool decode_uses_plan(const CacheGeom& g, const DecodeArgs& a) {
  const int64_t grid = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
  return a.num_seqs > 0 && a.num_partitions > 1 && a.seq_shared == nullptr && grid >= kPlanMinGrid;
}

hipError_t launch_decode_plan(const CacheGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (!decode_uses_plan(g, a)) return hipSuccess;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, plan_place(g, a));
  return hipGetLastError();
}

hipError_t launch_decode(const CacheGeom& g, int kind, const DecodeArgs& a, bool* supported,
                         hipStream_t stream, bool plan_made) {
  *supported = true;
  if (a.num_seqs <= 0) return hipSuccess;
  if (a.num_q_heads / g.num_kv_heads > kMaxGroup || (g.head_dim != 128 && g.head_dim != 64)) {
    *supported = false;
    return hipSuccess;
  }
  DecodeArgs ap = a;
  if (decode_uses_plan(g, a)) {
    if (!plan_made) {
      const hipError_t ep = launch_decode_plan(g, a, stream);
      if (ep != hipSuccess) return ep;
    }
    ap.plan = plan_place(g, a);
  }
  hipError_t e = hipSuccess;
  if (kind == kBF16 && g.head_dim == 128) e = launch_decode_bs<kBF16, 128>(g, ap, supported, stream);
  else if (kind == kBF16 && g.head_dim == 64) e = launch_decode_bs<kBF16, 64>(g, ap, supported, stream);
  else if (kind == kF32 && g.head_dim == 128) e = launch_decode_bs<kF32, 128>(g, ap, supported, stream);
  else if (kind == kF32 && g.head_dim == 64) e = launch_decode_bs<kF32, 64>(g, ap, supported, stream);
  else *supported = false;
  if (!*supported || e != hipSuccess || a.num_partitions == 1) return e;
  return g.head_dim == 128 ? launch_merge_d<128>(a, stream) : launch_merge_d<64>(a, stream);
}

}  // namespace pa
