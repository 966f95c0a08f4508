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
//     partition); the G query heads of the GQA group share every K/V load;
//   * waves take the partition's blocks round-robin; each (block, head) is
//     BS rows of head_dim elements, contiguous in memory, read with coalesced
//     16-byte loads: a row is LPR lanes, a wave instruction covers RPI rows;
//   * q.k: bf16 pairs through v_dot2_f32_bf16 (fp32 FMAs for fp32 caches),
//     then a butterfly over the LPR lanes of the row with DPP (quad_perm,
//     row_half_mirror, row_mirror) so every lane holds the same fp32 score;
//   * online softmax in fp32 with exp2 on pre-scaled scores; p*V in fp32;
//   * waves merge through LDS in a fixed order; partitions are merged by a
//     second small kernel in partition order.  Every reduction order depends
//     only on logical token positions, so results do not depend on which
//     physical blocks hold the tokens, nor on paged vs contiguous storage.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kMergeThreads = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Workgroups of a launch are dealt to the 8 XCDs round-robin by id.  Give
// each XCD one contiguous range of work items so that neighbours (partitions
// of one sequence, samples sharing a prompt's blocks) meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcd = 8;
  const int q = n / kXcd, rem = n % kXcd;
  const int x = bid % kXcd, local = bid / kXcd;
  return (x < rem) ? x * (q + 1) + local : rem * (q + 1) + (x - rem) * q + local;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane exchange inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;     // lane i <- 15-i
constexpr int kRowHalfMirror = 0x141; // lane i <- 7-i within each half row

// lane ^ M for M in {8, 16} (ds_swizzle bit mode, within 32 lanes) or 32.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  if constexpr (M < 32) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
  } else {
    return __shfl_xor(x, 32);
  }
}

// Sum over the LPR consecutive lanes of a token row; every lane of the row
// ends with the same bits (each step adds two equal-valued halves).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (LPR >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kRowMirror>(x);
  if constexpr (LPR >= 32) x += lane_xor<16>(x);
  return x;
}

// Combine the RPI rows of a wave (lanes that differ by multiples of LPR).
template <int LPR>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (LPR <= 8) x += lane_xor<8>(x);
  if constexpr (LPR <= 16) x += lane_xor<16>(x);
  if constexpr (LPR <= 32) x += lane_xor<32>(x);
  return x;
}
template <int LPR>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (LPR <= 8) x = fmaxf(x, lane_xor<8>(x));
  if constexpr (LPR <= 16) x = fmaxf(x, lane_xor<16>(x));
  if constexpr (LPR <= 32) x = fmaxf(x, lane_xor<32>(x));
  return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

// <q, k> over one 16-byte chunk.
template <int KIND>
__device__ __forceinline__ float dot16(const uint4& q, const uint4& k) {
  if constexpr (KIND == kBF16) {
    float x = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), 0.0f, false);
    x = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), x, false);
    x = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), x, false);
    x = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), x, false);
    return x;
  } else {
    float x = __uint_as_float(q.x) * __uint_as_float(k.x);
    x = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), x);
    x = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), x);
    x = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), x);
    return x;
  }
}

// 16-byte chunk to fp32 values (exact).
template <int KIND, int VE>
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[VE]) {
  if constexpr (KIND == kBF16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(w[k] << 16);
      f[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
}

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------------------
// decode: one workgroup per (sequence, KV head, partition)
// ---------------------------------------------------------------------------
template <int KIND, int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(CacheGeom geo, DecodeArgs a) {
  constexpr int ELT = KIND == kBF16 ? 2 : 4;
  constexpr int VE = 16 / ELT;      // elements per 16-byte chunk
  constexpr int LPR = D / VE;       // lanes per token row
  constexpr int RPI = kWave / LPR;  // token rows per wave instruction
  constexpr int NI = BS / RPI;      // wave instructions per block
  constexpr int ROW = D * ELT;      // bytes per (token, head) row
  constexpr int BLK = BS * ROW;     // bytes per (block, head)
  static_assert(LPR * VE == D && RPI * LPR == kWave && NI * RPI == BS && NI >= 1, "shape");

  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];

  const int P = a.num_partitions;
  const int hkv = geo.num_kv_heads;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int part = work % P;
  const int sk = work / P;
  const int kvh = sk % hkv;
  const int s = sk / hkv;
  const int tid = threadIdx.x;
  const int h0 = kvh * G;

  const int L = a.lens[s];
  const int nblk = (L + BS - 1) / BS;
  const int jb = part * a.partition_blocks;
  const int je = min(nblk, jb + a.partition_blocks);
  if (jb >= je) {
    if (P == 1) {  // empty context: zero output
      float* o = a.out + (static_cast<int64_t>(s) * a.num_q_heads + h0) * D;
      for (int e = tid; e < G * D; e += kThreads) o[e] = 0.0f;
    }
    return;
  }

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = lane / LPR;
  const int c = lane % LPR;

  uint4 qv[G];
  {
    const char* qb = static_cast<const char*>(a.q) +
                     (static_cast<int64_t>(s) * a.num_q_heads + h0) * ROW + c * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g] = ld16(qb + g * ROW);
  }
  const float c2 = a.scale * kLog2e;

  const char* kl = geo.k_base + static_cast<int64_t>(a.layer) * geo.layer_bytes + r * ROW + c * 16;
  const char* vl = geo.v_base + static_cast<int64_t>(a.layer) * geo.layer_bytes + r * ROW + c * 16;
  const int32_t* table = nullptr;
  int64_t seq_off = 0;
  if (geo.paged) {
    table = a.tables + static_cast<int64_t>(s) * a.table_stride;
  } else {
    const int rid = a.req_ids ? a.req_ids[s] : s;
    seq_off = (static_cast<int64_t>(rid) * hkv + kvh) * geo.unit * ROW;
  }
  auto block_off = [&](int j) -> int64_t {
    if (geo.paged) return (static_cast<int64_t>(table[j]) * hkv + kvh) * BLK;
    return seq_off + static_cast<int64_t>(j) * BLK;
  };

  float m[G], lsum[G], acc[G][VE];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;
  }

  uint4 kr[NI], vr[NI];
  int j = jb + wave;
  if (j < je) {
    const int64_t off = block_off(j);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = ld16(kl + off + i * RPI * ROW);
      vr[i] = ld16(vl + off + i * RPI * ROW);
    }
  }
  while (j < je) {
    const int jn = j + kWaves;
    uint4 kn[NI], vn[NI];
    if (jn < je) {
      const int64_t off = block_off(jn);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kn[i] = ld16(kl + off + i * RPI * ROW);
        vn[i] = ld16(vl + off + i * RPI * ROW);
      }
    }
    // scores of this lane's rows, pre-scaled to log2 units
    float sc[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) sc[i][g] = row_sum<LPR>(dot16<KIND>(qv[g], kr[i])) * c2;
    const int t0 = j * BS + r;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (t0 + i * RPI >= L)
#pragma unroll
        for (int g = 0; g < G; ++g) sc[i][g] = -INFINITY;
    // online softmax update
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = sc[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) bm = fmaxf(bm, sc[i][g]);
      bm = rows_max<LPR>(bm);
      const float mn = fmaxf(m[g], bm);
      const float alpha = fexp2(m[g] - mn);
      m[g] = mn;
      lsum[g] *= alpha;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float p = fexp2(sc[i][g] - mn);
        sc[i][g] = p;
        lsum[g] += p;
      }
    }
    // p * V
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[VE];
      unpack<KIND, VE>(vr[i], vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(sc[i][g], vf[e], acc[g][e]);
    }
    j = jn;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = kn[i];
      vr[i] = vn[i];
    }
  }

  // combine the rows of the wave, then the waves of the workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = rows_sum<LPR>(lsum[g]);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = rows_sum<LPR>(acc[g][e]);
  }
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VE; ++e) sm_acc[wave][g][c * VE + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[wave][g] = m[g];
      sm_l[wave][g] = lsum[g];
    }
  }
  __syncthreads();
  const int64_t row0 = static_cast<int64_t>(s) * a.num_q_heads + h0;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, e = idx % D;
    float mx = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][g]);
    float A = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fexp2(sm_m[w][g] - mx);
      A = fmaf(wt, sm_acc[w][g][e], A);
      Lt = fmaf(wt, sm_l[w][g], Lt);
    }
    if (P == 1) {
      a.out[(row0 + g) * D + e] = A / Lt;
    } else {
      const int64_t prow = (row0 + g) * P + part;
      float* acc_ws = a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads * P * 2;
      acc_ws[prow * D + e] = A;
      if (e == 0) {
        a.ws[prow * 2] = mx;
        a.ws[prow * 2 + 1] = Lt;
      }
    }
  }
}

// Merge context partitions in partition order: one workgroup per (seq, q head).
template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a, int block_size) {
  const int sh = blockIdx.x;
  const int s = sh / a.num_q_heads;
  const int P = a.num_partitions;
  const int L = a.lens[s];
  const int tp = a.partition_blocks * block_size;
  const int ps = (L + tp - 1) / tp;
  const float* ml = a.ws + static_cast<int64_t>(sh) * P * 2;
  const float* accp = a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads * P * 2 +
                      static_cast<int64_t>(sh) * P * D;
  float* o = a.out + static_cast<int64_t>(sh) * D;
  if (ps == 0) {
    for (int e = threadIdx.x; e < D; e += kMergeThreads) o[e] = 0.0f;
    return;
  }
  float mx = ml[0];
  for (int p = 1; p < ps; ++p) mx = fmaxf(mx, ml[2 * p]);
  for (int e = threadIdx.x; e < D; e += kMergeThreads) {
    float A = 0.0f, Lt = 0.0f;
    for (int p = 0; p < ps; ++p) {
      const float wt = fexp2(ml[2 * p] - mx);
      A = fmaf(wt, accp[p * D + e], A);
      Lt = fmaf(wt, ml[2 * p + 1], Lt);
    }
    o[e] = A / Lt;
  }
}

// ---------------------------------------------------------------------------
// append and copy-on-write copies
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kv_kernel(CacheGeom g, int32_t layer,
                                                        const uint4* __restrict__ k,
                                                        const uint4* __restrict__ v,
                                                        const int32_t* __restrict__ slots,
                                                        int32_t n) {
  const int chunks = g.head_dim * g.elt / 16;
  const int per_tok = g.num_kv_heads * chunks;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * per_tok) return;
  const int i = static_cast<int>(idx / per_tok);
  const int rem = static_cast<int>(idx % per_tok);
  const int h = rem / chunks, ch = rem % chunks;
  const int slot = slots[i];
  if (slot < 0) return;
  const int u = slot / g.unit, o = slot % g.unit;
  const int64_t dst = static_cast<int64_t>(layer) * g.layer_bytes +
                      ((static_cast<int64_t>(u) * g.num_kv_heads + h) * g.unit + o) *
                          (static_cast<int64_t>(g.head_dim) * g.elt) +
                      ch * 16;
  *reinterpret_cast<uint4*>(g.k_base + dst) = k[idx];
  *reinterpret_cast<uint4*>(g.v_base + dst) = v[idx];
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(CacheGeom g,
                                                          const int32_t* __restrict__ pairs) {
  const int pi = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
  const int64_t bb = static_cast<int64_t>(g.num_kv_heads) * g.block_size * g.head_dim * g.elt;
  const int64_t lb = static_cast<int64_t>(layer) * g.layer_bytes;
  const uint4* ks = reinterpret_cast<const uint4*>(g.k_base + lb + src * bb);
  const uint4* vs = reinterpret_cast<const uint4*>(g.v_base + lb + src * bb);
  uint4* kd = reinterpret_cast<uint4*>(g.k_base + lb + dst * bb);
  uint4* vd = reinterpret_cast<uint4*>(g.v_base + lb + dst * bb);
  for (int64_t x = threadIdx.x; x < bb / 16; x += 256) {
    kd[x] = ks[x];
    vd[x] = vs[x];
  }
}

template <int KIND, int D, int BS, int G>
hipError_t launch_decode_t(const CacheGeom& g, const DecodeArgs& a, hipStream_t st) {
  const int64_t nwork = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
  hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, G>), dim3(static_cast<uint32_t>(nwork)),
                     dim3(kThreads), 0, st, g, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(static_cast<uint32_t>(a.num_seqs) * a.num_q_heads),
                     dim3(kMergeThreads), 0, st, a, g.block_size);
  return hipGetLastError();
}

template <int KIND, int D, int BS>
hipError_t launch_decode_g(const CacheGeom& g, const DecodeArgs& a, int G, bool* ok,
                           hipStream_t st) {
  switch (G) {
    case 1: return launch_decode_t<KIND, D, BS, 1>(g, a, st);
    case 2: return launch_decode_t<KIND, D, BS, 2>(g, a, st);
    case 3: return launch_decode_t<KIND, D, BS, 3>(g, a, st);
    case 4: return launch_decode_t<KIND, D, BS, 4>(g, a, st);
    case 5: return launch_decode_t<KIND, D, BS, 5>(g, a, st);
    case 6: return launch_decode_t<KIND, D, BS, 6>(g, a, st);
    case 7: return launch_decode_t<KIND, D, BS, 7>(g, a, st);
    case 8: return launch_decode_t<KIND, D, BS, 8>(g, a, st);
    default: *ok = false; return hipSuccess;
  }
}

template <int KIND, int D>
hipError_t launch_decode_bs(const CacheGeom& g, const DecodeArgs& a, int G, bool* ok,
                            hipStream_t st) {
  switch (g.block_size) {
    case 8: return launch_decode_g<KIND, D, 8>(g, a, G, ok, st);
    case 16: return launch_decode_g<KIND, D, 16>(g, a, G, ok, st);
    case 32: return launch_decode_g<KIND, D, 32>(g, a, G, ok, st);
    default: *ok = false; return hipSuccess;
  }
}

}  // namespace

hipError_t launch_append(const CacheGeom& g, int32_t layer, const void* k, const void* v,
                         const int32_t* slots, int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = static_cast<int64_t>(n) * g.num_kv_heads * (g.head_dim * g.elt / 16);
  const uint32_t blocks = static_cast<uint32_t>((threads + 255) / 256);
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

hipError_t launch_decode(const CacheGeom& g, int kind, const DecodeArgs& a, bool* supported,
                         hipStream_t stream) {
  *supported = true;
  if (a.num_seqs <= 0) return hipSuccess;
  const int G = a.num_q_heads / g.num_kv_heads;
  if (kind == kBF16 && g.head_dim == 128) return launch_decode_bs<kBF16, 128>(g, a, G, supported, stream);
  if (kind == kBF16 && g.head_dim == 64) return launch_decode_bs<kBF16, 64>(g, a, G, supported, stream);
  if (kind == kF32 && g.head_dim == 128) return launch_decode_bs<kF32, 128>(g, a, G, supported, stream);
  if (kind == kF32 && g.head_dim == 64) return launch_decode_bs<kF32, 64>(g, a, G, supported, stream);
  *supported = false;
  return hipSuccess;
}

}  // namespace pa
