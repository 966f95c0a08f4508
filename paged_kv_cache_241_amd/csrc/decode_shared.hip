// Shared-prefix decode for gfx950.  Samples of one prompt point at the same
// physical blocks ("Efficient Memory Management for Large Language Model
// Serving with PagedAttention" summary page, Summary; "Running Out of Cache",
// "Fragmentation is lost users"): their attention over those blocks reads the
// same K and V.  This pass reads each shared chunk once per (group, KV head)
// and attends every member's query heads to it.
//
// One workgroup of 4 waves per (group, KV head, block of 64 query columns,
// partition of the shared prefix).  A query column is one (member, query
// head) pair; wave w owns columns 16w .. 16w + 15 of the block, the same
// 16-column MFMA tile the partition kernel uses for one sequence's heads.
// Per 16-token chunk the workgroup copies K and V once into LDS (double
// buffered, one barrier per chunk); every wave reads its operands from LDS in
// the lane layout of the partition kernel and runs the same score tile,
// online softmax and P V tiles over all chunks of the partition.  Each wave
// writes its columns' partials (running max, weight sum, unnormalised output)
// into the split-K workspace at the members' own partition slots; the
// partition kernel does the private partitions and the merge kernel combines
// them all in partition order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "decode_common.hpp"
#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kSharedWaves = 4;
constexpr int kColsPerWave = 16;
constexpr int kColsPerBlock = kSharedWaves * kColsPerWave;

template <int KIND, int D, int BS>
__global__ __launch_bounds__(kSharedWaves * kWave) void decode_shared_kernel(CacheGeom geo,
                                                                             DecodeArgs a,
                                                                             SharedArgs g) {
  using GG = Geo<KIND, D, BS>;
  constexpr int NX = GG::NX, NN = GG::NN, TILE = GG::TILE, ELT = GG::ELT;
  constexpr int kThreads = kSharedWaves * kWave;
  constexpr int kUnits = D * ELT;  // 16-byte units of one chunk's K, and of its V
  // two stage buffers of 2 chunks' K and V
  __shared__ __align__(16) char lds[2 * 2 * 2 * kUnits * 16];

  const int hkv = geo.num_kv_heads;
  int w = blockIdx.x;
  const int part = w % g.shared_parts;
  w /= g.shared_parts;
  const int cblk = w % g.col_blocks;
  w /= g.col_blocks;
  const int kvh = w % hkv;
  const int grp = w / hkv;
  const int first = g.groups[2 * grp];
  const int members = g.groups[2 * grp + 1];
  const int G = a.num_q_heads / hkv;
  const int ncols = members * G;
  const int shared = a.seq_shared[first];
  const int cb = part * a.partition_chunks;
  const int ce = min(cb + a.partition_chunks, shared / kChunk);
  if (cb >= ce || cblk * kColsPerBlock >= ncols) return;  // the whole workgroup

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15;
  const int j4 = lane >> 4;
  const int col0 = cblk * kColsPerBlock + wave * kColsPerWave;

  // q operand: column col0 + n = (member, head); columns past the group are
  // zero (their address is clamped to the group's last column)
  uint4 qop[NX];
  {
    const int col = min(col0 + n, ncols - 1);
    const int hq = kvh * G + col % G;
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(first + col / G) * a.num_q_heads + hq) * D) * ELT;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const uint4 v = ld16(qb + (x * 4 + j4) * 16);
      qop[x] = col0 + n < ncols ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const float c2 = a.scale * kLog2e;

  const char* kl = geo.k_base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  const char* vl = geo.v_base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  // the group's blocks are its first member's (all members hold the same ones)
  const const_i32_ptr table = reinterpret_cast<const_i32_ptr>(
      reinterpret_cast<uintptr_t>(a.tables + static_cast<int64_t>(first) * a.table_stride));

  // Stages of STEP consecutive chunks move through LDS.  Chunk j of a stage
  // is K as [D/VE pieces][16 rows][16 B] and V as [D][16 tokens] -- the tile
  // layouts of a 16-token block: unit uu < kUnits of a chunk's K is piece
  // uu/16, row uu%16; of its V, dim uu/ELT, tokens (uu%ELT)*16/ELT on.  The
  // next stage's loads are in flight while a stage is computed, and one
  // barrier and one softmax step serve STEP chunks: a stage's critical path
  // (LDS write, barrier, LDS read, the score tile, the max reduction, the P V
  // tiles) is what bounds this kernel, not its memory traffic.
  constexpr int STEP = 2;
  constexpr int kStage = STEP * kUnits;  // 16-byte units of a stage's K (and of its V)
  constexpr int kPerS = (kStage + kThreads - 1) / kThreads;
  constexpr int kStageBuf = 2 * kStage * 16;
  static_assert(2 * kStageBuf <= static_cast<int>(sizeof(lds)), "LDS stage buffers");
  uint4 sk[kPerS], sv[kPerS];
  // stage st of the partition: chunks cb + st*STEP + j, clamped into the
  // partition (the clamped copies are masked out below)
  auto load_stage = [&](int st) {
#pragma unroll
    for (int k = 0; k < kPerS; ++k) {
      const int u = tid + k * kThreads;
      if (kPerS * kThreads == kStage || u < kStage) {
        const int uu = u % kUnits;
        const int c = min(cb + st * STEP + u / kUnits, ce - 1);
        const int t = c * kChunk + uu % 16;
        const int tv = c * kChunk + (uu % ELT) * (16 / ELT);
        int64_t bk, bv;
        if constexpr (BS >= kChunk) {
          bk = bv = static_cast<int64_t>(table[(c * kChunk) / BS]);
        } else {
          bk = static_cast<int64_t>(table[t / BS]);
          bv = static_cast<int64_t>(table[tv / BS]);
        }
        sk[k] = ld16(kl + (bk * hkv + kvh) * TILE + ((uu / 16) * BS + t % BS) * 16);
        sv[k] = ld16(vl + (bv * hkv + kvh) * TILE + ((uu / ELT) * BS + tv % BS) * ELT);
      }
    }
  };
  auto store_stage = [&](int buf) {
    char* kd = lds + buf * kStageBuf;
    char* vd = kd + kStage * 16;
#pragma unroll
    for (int k = 0; k < kPerS; ++k) {
      const int u = tid + k * kThreads;
      if (kPerS * kThreads == kStage || u < kStage) {
        *reinterpret_cast<uint4*>(kd + u * 16) = sk[k];
        *reinterpret_cast<uint4*>(vd + u * 16) = sv[k];
      }
    }
  };

  float m = -INFINITY;
  float lsum = 0.0f;
  floatx4_t acc[NN];
#pragma unroll
  for (int nb = 0; nb < NN; ++nb) acc[nb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int stages = (ce - cb + STEP - 1) / STEP;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < stages; ++st) {
    const int buf = st & 1;
    // loads past the last stage re-read the partition's last chunk (an L2
    // hit) rather than branch: a branch around loads makes the wait for them
    // also wait for every newer load
    load_stage(min(st + 1, stages - 1));
    const char* kd = lds + buf * kStageBuf;
    const char* vd = kd + kStage * 16;
    // S[j][token 4*j4+i][column n]: the score tiles of the stage's chunks
    floatx4_t S[STEP];
#pragma unroll
    for (int j = 0; j < STEP; ++j) {
      S[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const uint4 kop =
            *reinterpret_cast<const uint4*>(kd + j * kUnits * 16 + ((x * 4 + j4) * 16 + n) * 16);
        if constexpr (KIND == kBF16) {
          S[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop),
                                                         __builtin_bit_cast(bf16x8_t, qop[x]), S[j], 0, 0, 0);
        } else {
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop.x), __uint_as_float(qop[x].x), S[j], 0, 0, 0);
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop.y), __uint_as_float(qop[x].y), S[j], 0, 0, 0);
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop.z), __uint_as_float(qop[x].z), S[j], 0, 0, 0);
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop.w), __uint_as_float(qop[x].w), S[j], 0, 0, 0);
        }
      }
    }
    // one online-softmax step for column n over the stage's chunks; chunks
    // past the partition (clamped copies) weigh nothing
    float sc[STEP][4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < STEP; ++j) {
      const bool live = cb + st * STEP + j < ce;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[j][i] = live ? S[j][i] * c2 : -INFINITY;
        mx = fmaxf(mx, sc[j][i]);
      }
    }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float mn = fmaxf(m, mx);
    const float alpha = fexp2(m - mn);
    m = mn;
    if (__any(alpha != 1.0f)) {
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j4 + i);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= ai[i];
    }
    float part_sum = 0.0f;
#pragma unroll
    for (int j = 0; j < STEP; ++j) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fexp2(sc[j][i] - mn);
      const char* vj = vd + j * kUnits * 16;
      if constexpr (KIND == kBF16) {
        const uint32_t hi01 = pack_bf16(p[0], p[1]), hi23 = pack_bf16(p[2], p[3]);
        const float h0f = bf16_lo(hi01), h1f = bf16_hi(hi01), h2f = bf16_lo(hi23), h3f = bf16_hi(hi23);
        const uint32_t lo01 = pack_bf16(p[0] - h0f, p[1] - h1f), lo23 = pack_bf16(p[2] - h2f, p[3] - h3f);
        part_sum += ((h0f + bf16_lo(lo01)) + (h1f + bf16_hi(lo01))) +
                    ((h2f + bf16_lo(lo23)) + (h3f + bf16_hi(lo23)));
        const short4_t phi = __builtin_bit_cast(short4_t, make_uint2(hi01, hi23));
        const short4_t plo = __builtin_bit_cast(short4_t, make_uint2(lo01, lo23));
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
          const uint2 vop = *reinterpret_cast<const uint2*>(vj + ((nb * 16 + n) * 16 + 4 * j4) * ELT);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, __builtin_bit_cast(short4_t, vop),
                                                             acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, __builtin_bit_cast(short4_t, vop),
                                                             acc[nb], 0, 0, 0);
        }
      } else {
        part_sum += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
          const uint4 vop = *reinterpret_cast<const uint4*>(vj + ((nb * 16 + n) * 16 + 4 * j4) * ELT);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], __uint_as_float(vop.x), acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], __uint_as_float(vop.y), acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], __uint_as_float(vop.z), acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], __uint_as_float(vop.w), acc[nb], 0, 0, 0);
        }
      }
    }
    lsum = lsum * alpha + part_sum;
    store_stage(buf ^ 1);
    __syncthreads();
  }

  // partials of this wave's columns at the members' partition slot `part`
  lsum += xor16(lsum);
  lsum += xor32(lsum);
  const int P = a.num_partitions;
  float* acc_ws = a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads * P * 2;
  auto prow = [&](int col) -> int64_t {
    const int64_t row = static_cast<int64_t>(first + col / G) * a.num_q_heads + kvh * G + col % G;
    return row * P + part;
  };
  if (j4 == 0 && col0 + n < ncols) {
    const int64_t r = prow(col0 + n);
    a.ws[r * 2] = m;
    a.ws[r * 2 + 1] = lsum;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = col0 + 4 * j4 + i;
    if (col < ncols) {
      const int64_t r = prow(col);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) acc_ws[r * D + nb * 16 + n] = acc[nb][i];
    }
  }
}

template <int KIND, int D>
hipError_t launch_shared_d(const CacheGeom& g, const DecodeArgs& a, const SharedArgs& sh,
                           bool* supported, hipStream_t st) {
  const int64_t nwork =
      static_cast<int64_t>(sh.num_groups) * g.num_kv_heads * sh.col_blocks * sh.shared_parts;
  if (nwork == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(nwork)), block(kSharedWaves * kWave);
  switch (g.block_size) {
    case 8: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 8>), grid, block, 0, st, g, a, sh); break;
    case 16: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 16>), grid, block, 0, st, g, a, sh); break;
    case 32: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 32>), grid, block, 0, st, g, a, sh); break;
    default: *supported = false; return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_shared(const CacheGeom& g, int kind, const DecodeArgs& a,
                                const SharedArgs& sh, bool* supported, hipStream_t stream) {
  *supported = true;
  if (a.num_q_heads / g.num_kv_heads > kColsPerWave) {
    *supported = false;
    return hipSuccess;
  }
  if (kind == kBF16 && g.head_dim == 128) return launch_shared_d<kBF16, 128>(g, a, sh, supported, stream);
  if (kind == kBF16 && g.head_dim == 64) return launch_shared_d<kBF16, 64>(g, a, sh, supported, stream);
  if (kind == kF32 && g.head_dim == 128) return launch_shared_d<kF32, 128>(g, a, sh, supported, stream);
  if (kind == kF32 && g.head_dim == 64) return launch_shared_d<kF32, 64>(g, a, sh, supported, stream);
  *supported = false;
  return hipSuccess;
}

}  // namespace pa
