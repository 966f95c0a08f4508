// Shared-prefix decode for gfx950.  Samples of one prompt point at the same
// physical blocks ("Efficient Memory Management for Large Language Model
// Serving with PagedAttention" summary page, Summary; "Running Out of Cache",
// "Fragmentation is lost users"): their attention over those blocks reads the
// same K and V.  This pass reads each shared chunk once per (group, KV head)
// and attends every member's query heads to it.
//
// One workgroup of 8 waves per (group, KV head, block of 64 query columns,
// partition of the shared prefix).  A query column is one (member, query
// head) pair.  The waves form two sets of 4; in each set wave w owns columns
// 16w .. 16w + 15 of the block, the same 16-column MFMA tile the partition
// kernel uses for one sequence's heads.  Per stage of four 16-token chunks
// (two for fp32) the workgroup copies K and V once into LDS (double
// buffered, one barrier per stage); set s reads the stage's chunks 2s and
// 2s + 1 from LDS and runs the score tiles, one online-softmax step and the
// P V products.  At the end the second set's state merges into the first's,
// which writes its columns' partials (running max, weight sum, unnormalised
// output) into the split-K workspace at the members' own partition slots.
// The rest of the launch runs the partition kernel's body for the private
// partitions, two work items per workgroup (one per set of 4 waves), and the
// merge kernel combines all partitions in partition order.
//
// What bounds it (measured on MI355X): the shared pass's per-stage chain
// (load -> LDS -> score tiles, softmax, P V) more than HBM; two sets per
// workgroup keep twice the loads in flight and halve the stages, which
// shortened the Yi-6B shared-prefix step from 84.4 to 83.6 us per layer
// (one set per 4-wave workgroup and 4-wave partition workgroups before).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "decode_common.hpp"
#include "decode_partition.hpp"
#include "kernels.hpp"

namespace pa {
namespace {

// Two sets of 4 waves: the 4 waves of a set own the block's 64 query
// columns, 16 each, and the two sets attend to different chunks of every
// stage; their online-softmax states are merged at the end.
constexpr int kSets = 2;
constexpr int kSetWaves = 4;
constexpr int kSharedWaves = kSets * kSetWaves;
constexpr int kColsPerWave = 16;
constexpr int kColsPerBlock = kSetWaves * kColsPerWave;

// max over lanes l, l ^ 16 and l ^ 32 with the cross-lane swaps of the VALU
// (v_permlane16_swap: rows 1 and 3 of the first operand trade places with
// rows 0 and 2 of the second; v_permlane32_swap: the upper half of the first
// with the lower half of the second).  Swapping x with itself leaves x[l] in
// one result and x[l ^ 16] (x[l ^ 32]) in the other, in every lane.
__device__ __forceinline__ float max_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

// Chunks per set and stage of the shared pass: two for bf16 (one 32-token
// P V step), one for fp32 (which keeps the two stage buffers at 66 KiB).
template <int KIND>
constexpr int shared_step() { return KIND == kBF16 ? 2 : 1; }
// LDS bytes of the shared pass: two stage buffers, each one part per set
// (see below)
template <int KIND, int D>
constexpr int shared_lds_bytes() {
  constexpr int ELT = KIND == kBF16 ? 2 : 4, STEP = shared_step<KIND>();
  return 2 * kSets * (STEP * D * ELT * 16 + 4 * (D * 4 * ELT * STEP + 128));
}

// The shared pass of workgroup w, with `lds` shared_lds_bytes() of LDS.
template <int KIND, int D, int BS>
__device__ __forceinline__ void shared_pass(const CacheGeom& geo, const DecodeArgs& a, const SharedArgs& g,
                                            int w, char* lds) {
  using GG = Geo<KIND, D, BS>;
  constexpr int NX = GG::NX, NN = GG::NN, CH = GG::CH, SUBPAIR = GG::SUBPAIR, PAIR = GG::PAIR, ELT = GG::ELT;
  constexpr int kThreads = kSharedWaves * kWave;
  constexpr int kUnits = D * ELT;  // 16-byte units of one chunk's K, and of its V
  // Stages of SCH consecutive chunks move through LDS (double buffered):
  // set s attends to chunks s*STEP .. s*STEP + STEP-1 of each stage, held in
  // its own part of the stage buffer.  K keeps the tile layout, [D/VE
  // pieces][16 rows][16 B] per chunk: the score operands of a wave are 1 KiB
  // contiguous reads.  V is regrouped: record (token group j4, dim e) holds
  // tokens 4*j4 .. 4*j4+3 of dim e of each of the set's chunks, chunk after
  // chunk, so that a lane's P V operand is one 16-byte read and the 16 lanes
  // of a token group read 256 contiguous bytes (no bank conflicts); the four
  // token groups are padded apart by 128 bytes.  For bf16 the two chunks of a
  // set form one 32-token P V step of v_mfma_f32_16x16x32_bf16, token (chunk
  // j, 4*j4+i) being k index 8*j4 + 4*j + i of both operands.
  constexpr int STEP = shared_step<KIND>();
  constexpr int SCH = kSets * STEP;       // chunks of a stage
  constexpr int kSetUnits = STEP * kUnits;  // 16-byte units of a set's K (and of its V) per stage
  constexpr int kStage = SCH * kUnits;      // 16-byte units of a stage's K (and of its V)
  constexpr int kVRec = 4 * ELT * STEP;
  constexpr int kVSeg = D * kVRec + 128;
  constexpr int kKBytes = kSetUnits * 16;
  constexpr int kSetBuf = kKBytes + 4 * kVSeg;
  constexpr int kStageBuf = kSets * kSetBuf;
  static_assert(KIND != kBF16 || kVRec == 16, "a bf16 record is one 32-token operand");
  static_assert(2 * kStageBuf == shared_lds_bytes<KIND, D>(), "LDS stage buffers");

  const int hkv = geo.num_kv_heads;
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
  const int set = wave / kSetWaves;   // which chunks of a stage
  const int cw = wave % kSetWaves;    // which 16 columns
  const int n = lane & 15;
  const int j4 = lane >> 4;
  const int col0 = cblk * kColsPerBlock + cw * kColsPerWave;

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

  // K tiles of the layer; each V tile follows its K tile
  const char* kl = geo.base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  const char* vl = kl + CH;
  // the group's blocks are its first member's (all members hold the same ones)
  const const_i32_ptr table = reinterpret_cast<const_i32_ptr>(
      reinterpret_cast<uintptr_t>(a.tables + static_cast<int64_t>(first) * a.table_stride));

  // Thread u of the workgroup moves units u, u + kThreads, ... of a stage:
  // unit uu < kUnits of chunk j is K piece uu/16, row uu%16, and V dim uu/ELT,
  // tokens (uu%ELT)*16/ELT on.  kUnits is a multiple of the wave, so a
  // unit's chunk j is wave-uniform, and with blocks of at least a chunk its
  // table entry is a scalar load.  The next stage's loads are in flight while
  // a stage is computed; one barrier and one softmax step serve STEP chunks.
  // Each shared chunk is read once per launch, so the loads are non-temporal
  // (84 against 85 us on the Yi-6B shared-prefix workload): they leave the
  // caches to the private partitions running beside this pass.
  constexpr int kPerS = (kStage + kThreads - 1) / kThreads;
  static_assert(kUnits % kWave == 0, "a wave's units lie in one chunk");
  // chunk of the stage that unit tid + k*kThreads belongs to
  auto chunk_of = [&](int k) -> int {
    if constexpr (kUnits % kThreads == 0) return (k * kThreads) / kUnits;
    else return __builtin_amdgcn_readfirstlane((wave * kWave + k * kThreads) / kUnits);
  };
  // the lane's offsets of its units inside a chunk's tile pair, for blocks
  // of at least a chunk (the pair's place in its block is wave-uniform)
  uint32_t ko[kPerS], vo[kPerS];
#pragma unroll
  for (int k = 0; k < kPerS; ++k) {
    const int uu = tid + k * kThreads - chunk_of(k) * kUnits;
    ko[k] = static_cast<uint32_t>(uu * 16);
    vo[k] = static_cast<uint32_t>(((uu / ELT) * kChunk + (uu % ELT) * (16 / ELT)) * ELT);
  }
  uint4 sk[kPerS], sv[kPerS];
  // stage st of the partition: chunks cb + st*SCH + j, clamped into the
  // partition (the clamped copies are masked out below).  past: the stage
  // after the last, loaded only so that the loop needs no branch around its
  // loads (a branch makes the wait for them also wait for every newer load);
  // all lanes then read the first 16 bytes of the partition's first chunk,
  // one line per wave instead of a stage of chunks from HBM again.
  auto load_stage = [&](int st, bool past, uint4 (&sk)[kPerS], uint4 (&sv)[kPerS]) {
    if constexpr (BS >= kChunk) {
      const char* kb[SCH];
      const char* vb[SCH];
#pragma unroll
      for (int j = 0; j < SCH; ++j) {
        const int c = past ? cb : min(cb + st * SCH + j, ce - 1);
        const int64_t blk = table[__builtin_amdgcn_readfirstlane((c * kChunk) / BS)];
        const int64_t tile = (blk * hkv + kvh) * PAIR + ((c * kChunk) % BS / kChunk) * SUBPAIR;
        kb[j] = kl + tile;
        vb[j] = vl + tile;
      }
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        if (kPerS * kThreads == kStage || tid + k * kThreads < kStage) {
          const int j = chunk_of(k);
          const char* kbj = kb[0];
          const char* vbj = vb[0];
#pragma unroll
          for (int jj = 1; jj < SCH; ++jj) {
            kbj = j == jj ? kb[jj] : kbj;
            vbj = j == jj ? vb[jj] : vbj;
          }
          // a wave-uniform base plus a 32-bit lane offset (kept a 32-bit
          // value by the empty asm): the loads take the scalar-base form
          uint32_t ok = past ? 0u : ko[k], ov = past ? 0u : vo[k];
          asm volatile("" : "+v"(ok), "+v"(ov));
          sk[k] = kv16<true>(kbj + ok);
          sv[k] = kv16<true>(vbj + ov);
        }
      }
    } else {
      // 8-token blocks: a chunk spans two blocks, whose table entries are
      // wave-uniform scalar loads (the shared prefix is whole chunks, so both
      // lie in it); each unit takes its token's
      static_assert(2 * BS == kChunk, "blocks shorter than a chunk are half a chunk");
#pragma unroll
      for (int k = 0; k < kPerS; ++k) {
        const int u = tid + k * kThreads;
        if (kPerS * kThreads == kStage || u < kStage) {
          const int j = chunk_of(k);
          const int uu = past ? 0 : u - j * kUnits;
          const int c = past ? cb : min(cb + st * SCH + j, ce - 1);
          const int j0 = __builtin_amdgcn_readfirstlane(2 * c);
          const int64_t b0 = table[j0], b1 = table[j0 + 1];
          const int r = uu % 16;                     // K: the unit's token in the chunk
          const int rv = (uu % ELT) * (16 / ELT);    // V: its first token
          const int64_t bk = r < BS ? b0 : b1, bv = rv < BS ? b0 : b1;
          sk[k] = kv16<true>(kl + (bk * hkv + kvh) * PAIR + ((uu / 16) * BS + r % BS) * 16);
          sv[k] = kv16<true>(vl + (bv * hkv + kvh) * PAIR + ((uu / ELT) * BS + rv % BS) * ELT);
        }
      }
    }
  };
  auto store_stage = [&](int buf, const uint4 (&sk)[kPerS], const uint4 (&sv)[kPerS]) {
#pragma unroll
    for (int k = 0; k < kPerS; ++k) {
      const int u = tid + k * kThreads;
      if (kPerS * kThreads == kStage || u < kStage) {
        const int jc = chunk_of(k);      // chunk of the stage
        const int s = jc / STEP, j = jc % STEP;  // its set, and its place there
        char* kd = lds + buf * kStageBuf + s * kSetBuf;
        char* vd = kd + kKBytes;
        *reinterpret_cast<uint4*>(kd + (u - s * kSetUnits) * 16) = sk[k];
        const int uu = u - jc * kUnits;
        const int e = uu / ELT, q = uu % ELT;
        if constexpr (KIND == kBF16) {
          // tokens 8q .. 8q+7: token groups 2q and 2q+1
          *reinterpret_cast<uint2*>(vd + (2 * q) * kVSeg + e * kVRec + j * 8) = make_uint2(sv[k].x, sv[k].y);
          *reinterpret_cast<uint2*>(vd + (2 * q + 1) * kVSeg + e * kVRec + j * 8) = make_uint2(sv[k].z, sv[k].w);
        } else {
          // tokens 4q .. 4q+3: token group q
          *reinterpret_cast<uint4*>(vd + q * kVSeg + e * kVRec + j * 16) = sv[k];
        }
      }
    }
  };

  // acc[nb][i] = O[dim nb*16 + 4*j4 + i][column n]: the P V product is taken
  // as V^T P^T, so a column's rescale factor is its own lane's
  float m = -INFINITY;
  float lsum = 0.0f;
  floatx4_t acc[NN];
#pragma unroll
  for (int nb = 0; nb < NN; ++nb) acc[nb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Two stages in flight: while stage st is computed from LDS buffer st % 2,
  // stage st + 1 is loaded into registers; it goes to the other buffer after
  // the compute.  (A third stage in flight, in a second register set, was
  // measured slower: it costs occupancy and the wait is not the bound.)
  const int stages = (ce - cb + SCH - 1) / SCH;
  // one online-softmax step and the P V products of the set's chunks of the
  // stage in LDS buffer buf
  auto compute = [&](int buf, int st) {
    const char* kd = lds + buf * kStageBuf + set * kSetBuf;
    const char* vd = kd + kKBytes;
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
    // one online-softmax step for column n over the set's chunks; chunks
    // past the partition (clamped copies) weigh nothing
    float sc[STEP][4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < STEP; ++j) {
      const bool live = cb + st * SCH + set * STEP + j < ce;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[j][i] = live ? S[j][i] * c2 : -INFINITY;
        mx = fmaxf(mx, sc[j][i]);
      }
    }
    mx = max_rows(mx);
    const float mn = fmaxf(m, mx);
    // a set whose chunks have all been past the partition so far keeps
    // m = -inf and weighs nothing (mr avoids -inf - -inf)
    const float mr = mn == -INFINITY ? 0.0f : mn;
    const float alpha = fexp2(m - mr);
    m = mn;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= alpha;
    }
    float p[STEP][4];
#pragma unroll
    for (int j = 0; j < STEP; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[j][i] = fexp2(sc[j][i] - mr);
    float part_sum = 0.0f;
    if constexpr (KIND == kBF16) {
      // weight = high + low, both bf16; the sum is what the MFMA multiplies
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < STEP; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float a0 = p[j][2 * h], a1 = p[j][2 * h + 1];
          const uint32_t wh = pack_bf16(a0, a1);
          const float h0 = bf16_lo(wh), h1 = bf16_hi(wh);
          const uint32_t wl = pack_bf16(a0 - h0, a1 - h1);
          part_sum += (h0 + bf16_lo(wl)) + (h1 + bf16_hi(wl));
          hi[2 * j + h] = wh;
          lo[2 * j + h] = wl;
        }
      }
      const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        const uint4 vop = *reinterpret_cast<const uint4*>(vd + j4 * kVSeg + (nb * 16 + n) * kVRec);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop), phi, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vop), plo, acc[nb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < STEP; ++j) {
        part_sum += (p[j][0] + p[j][1]) + (p[j][2] + p[j][3]);
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
          const uint4 vop = *reinterpret_cast<const uint4*>(vd + j4 * kVSeg + (nb * 16 + n) * kVRec + j * 16);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vop.x), p[j][0], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vop.y), p[j][1], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vop.z), p[j][2], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vop.w), p[j][3], acc[nb], 0, 0, 0);
        }
      }
    }
    lsum = lsum * alpha + part_sum;
  };
  load_stage(0, false, sk, sv);
  store_stage(0, sk, sv);
  __syncthreads();
  for (int st = 0; st < stages; ++st) {
    load_stage(st + 1, st + 1 >= stages, sk, sv);
    compute(st & 1, st);
    store_stage((st & 1) ^ 1, sk, sv);
    __syncthreads();
  }

  // the second set's state of the same columns, into the first set's
  // (the stage buffers are free after the loop's last barrier); per lane the
  // two states cover disjoint chunks, so they merge as two partitions do
  {
    constexpr int R = 2 + 4 * NN;
    static_assert(kSetWaves * R * kWave * 4 <= 2 * kStageBuf, "set merge fits the stage buffers");
    float* xf = reinterpret_cast<float*>(lds) + cw * R * kWave + lane;
    if (set == 1) {
      xf[0] = m;
      xf[kWave] = lsum;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[(2 + 4 * nb + i) * kWave] = acc[nb][i];
    }
    __syncthreads();
    if (set == 1) return;
    // the first set's first chunk lies in the partition: m is finite
    const float m1 = xf[0];
    const float mn = fmaxf(m, m1);
    const float a0 = fexp2(m - mn), a1 = fexp2(m1 - mn);
    m = mn;
    lsum = lsum * a0 + xf[kWave] * a1;
#pragma unroll
    for (int nb = 0; nb < NN; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nb][i] = acc[nb][i] * a0 + xf[(2 + 4 * nb + i) * kWave] * a1;
  }

  // partials of this wave's columns at the members' partition slot `part`
  lsum += xor16(lsum);
  lsum += xor32(lsum);
  if (col0 + n < ncols) {
    const int P = a.num_partitions;
    const int col = col0 + n;
    const int64_t r = (static_cast<int64_t>(first + col / G) * a.num_q_heads + kvh * G + col % G) * P + part;
    if (j4 == 0) {
      a.ws[r * 2] = m;
      a.ws[r * 2 + 1] = lsum;
    }
    float* o = a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads * P * 2 + r * D + 4 * j4;
#pragma unroll
    for (int nb = 0; nb < NN; ++nb)
      *reinterpret_cast<float4*>(o + nb * 16) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
  }
}

// One launch: workgroups [0, n_shared) do the shared pass, the rest the
// private partitions (the partition kernel's body, whose workgroups for
// shared partitions exit at once).  Both kinds are resident together, so
// the shared pass's compute overlaps the private partitions' HBM stream.
template <int KIND, int D, int BS>
__global__ __launch_bounds__(kSharedWaves * kWave)
__attribute__((amdgpu_waves_per_eu(decode_min_waves_per_eu<KIND, BS>())))
void decode_shared_kernel(CacheGeom geo, DecodeArgs a, SharedArgs g) {
  extern __shared__ __align__(16) char lds_dyn[];
  const int bid = blockIdx.x;
  if (bid < g.n_shared) {
    shared_pass<KIND, D, BS>(geo, a, g, bid, lds_dyn);
  } else {
    // two partition work items per workgroup, one per set of 4 waves, each
    // with its own LDS; every wave passes exactly one barrier (the body's
    // merge, or the one an idle half passes here)
    const int half = static_cast<int>(threadIdx.x) / (kSetWaves * kWave);
    const int item = 2 * (bid - g.n_shared) + half;
    if (item >= g.n_private) {
      __syncthreads();
      return;
    }
    decode_partition_body<KIND, D, BS, kSetWaves, true, false, false, true>(
        geo, a, item, g.n_private, reinterpret_cast<float*>(lds_dyn + half * g.private_lds));
  }
}

template <int KIND, int D>
hipError_t launch_shared_d(const CacheGeom& g, const DecodeArgs& a, const SharedArgs& sh,
                           bool* supported, hipStream_t st) {
  const int64_t n_private = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
  const int64_t nwork = static_cast<int64_t>(sh.n_shared) + (n_private + 1) / 2;
  if (nwork == 0) return hipSuccess;
  const int G = a.num_q_heads / g.num_kv_heads;
  // the shared pass's stage buffers, or two partition items' merge areas
  // (and, with a fused append, their staged tail chunks), whichever is larger
  const int private_lds = (merge_lds_bytes(kSetWaves, G, D) +
                           (a.new_k != nullptr ? append_lds_bytes(D, g.elt, g.block_size) : 0) + 15) /
                          16 * 16;
  const size_t lds = static_cast<size_t>(std::max(shared_lds_bytes<KIND, D>(), 2 * private_lds));
  SharedArgs sh2 = sh;
  sh2.n_private = static_cast<int32_t>(n_private);
  sh2.private_lds = private_lds;
  const dim3 grid(static_cast<uint32_t>(nwork)), block(kSharedWaves * kWave);
  switch (g.block_size) {
    case 8: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 8>), grid, block, lds, st, g, a, sh2); break;
    case 16: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 16>), grid, block, lds, st, g, a, sh2); break;
    case 32: hipLaunchKernelGGL((decode_shared_kernel<KIND, D, 32>), grid, block, lds, st, g, a, sh2); break;
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
