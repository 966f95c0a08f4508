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
//     physical blocks hold the tokens, nor on paged vs contiguous storage.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "decode_common.hpp"
#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kMergeWaves = 4;   // merge rows per workgroup, one a wave
constexpr int kMaxGroup = 16;     // query heads per KV head the tile can hold
constexpr int kMaxMergeLds = 64 * 1024;

// ---------------------------------------------------------------------------
// decode: one workgroup per (sequence, KV head, partition)
// ---------------------------------------------------------------------------
// bf16 caches with blocks of at least a chunk fit 128 VGPRs, i.e. four waves
// per SIMD (the occupancy the HBM stream needs); the others would spill.
template <int KIND, int BS>
constexpr int decode_min_waves_per_eu() { return KIND == kBF16 && BS >= kChunk ? 4 : 1; }
// LDS bytes of the wave merge: per wave, G maxima, G sums and G x D partial
// outputs.
__host__ __device__ constexpr int merge_lds_bytes(int waves, int G, int D) {
  return waves * G * (D + 2) * 4;
}

template <int KIND, int D, int BS, int W, bool NT>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(decode_min_waves_per_eu<KIND, BS>())))
void decode_partition_kernel(CacheGeom geo, DecodeArgs a) {
  using GG = Geo<KIND, D, BS>;
  constexpr int NX = GG::NX, NN = GG::NN, TILE = GG::TILE, ELT = GG::ELT;
  constexpr int kWaves = W;
  constexpr int kThreads = W * kWave;
  // V operand per lane per output tile: 4 consecutive tokens of one dim
  using VOp = typename std::conditional<KIND == kBF16, uint2, uint4>::type;

  const int P = a.num_partitions;
  const int hkv = geo.num_kv_heads;
  const int G = a.num_q_heads / hkv;
  // With a plan (split contexts), workgroup i takes the KV head i % hkv of
  // plan item i / hkv; the items with work fill the front of the grid,
  // longest first, and the grid's tail exits at once.  Without one (one
  // partition per context), work items are (r, sequence, KV head) with r a
  // partition's place counted from the end of its context, r-major and
  // descending; with one partition that is each context's only one.
  const int tid = threadIdx.x;
  int s, kvh, part, L;
  if (a.plan != nullptr) {
    const int2 it = a.plan[blockIdx.x / hkv];
    if (it.x < 0) return;
    s = it.x / P;
    part = it.x % P;
    kvh = blockIdx.x % hkv;
    L = it.y;
  } else {
    const int work = work_item(blockIdx.x, gridDim.x, !NT);
    const int pairs = a.num_seqs * hkv;
    const int r = P - 1 - work / pairs;
    kvh = (work % pairs) % hkv;
    s = (work % pairs) / hkv;
    L = a.lens[s];
    // partitions holding tokens (at most P: contexts are at most max_context)
    const int np = min((L + a.partition_chunks * kChunk - 1) / (a.partition_chunks * kChunk), P);
    part = np - 1 - r;
    if (part < 0) {
      if (P == 1) {  // empty context: zero output
        float* o = a.out + (static_cast<int64_t>(s) * a.num_q_heads + kvh * G) * D;
        for (int e = tid; e < G * D; e += kThreads) o[e] = 0.0f;
      }
      return;
    }
  }
  const int h0 = kvh * G;
  const int nch = (L + kChunk - 1) / kChunk;
  const int cb = part * a.partition_chunks;
  const int ce = min(nch, cb + a.partition_chunks);
  if (a.seq_shared != nullptr && cb * kChunk < a.seq_shared[s]) return;  // the shared pass's

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15;   // head column of S / row of the K tile
  const int j4 = lane >> 4;  // lane group: tokens 4*j4 .. 4*j4+3

  // Wave w takes chunks ce-1-w, ce-1-w-W, ... down to cb.  The last chunk of
  // the context, the only one that may be partly filled and the one that
  // holds the appended token, is then the first chunk of wave 0.
  //
  // Fused append: token L-1 arrives in new_k / new_v.  Wave 0 loads the row
  // into registers next to q, so its latency overlaps everything up to the
  // first chunk, where selects put it into the operand registers; it keeps a
  // copy in LDS and stores the row into the cache after its loop.  (Narrow
  // row stores at the end cost less than writing the whole chunk back from
  // the operand registers, whose writes would interleave with the reads.)
  // The row and the slot are loaded whatever the slot says: only their use
  // waits for the slot (a slot < 0 appends nothing and the cache is read as
  // it is), so no load of the workgroup's start waits on another.
  constexpr int kRowVec = D * ELT / 16;  // 16-byte pieces of one row
  __shared__ uint4 sm_new[2 * kRowVec];  // K pieces, then V pieces
  const bool last_new = a.new_k != nullptr && wave == 0 && ce == nch;
  int slot_new = -1;
  uint4 nk[NX];      // lane (n, j4): K pieces x*4+j4 of the new row
  uint32_t nv[NN];   // lane (n, j4): V element nb*16+n of the new row
  if (last_new) {
    slot_new = a.new_slots[s];
    const int64_t src = (static_cast<int64_t>(s) * hkv + kvh) * D * ELT;
    const char* nk_row = static_cast<const char*>(a.new_k) + src;
    const char* nv_row = static_cast<const char*>(a.new_v) + src;
#pragma unroll
    for (int x = 0; x < NX; ++x) nk[x] = ld16(nk_row + (x * 4 + j4) * 16);
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) {
      if constexpr (KIND == kBF16) nv[nb] = *reinterpret_cast<const uint16_t*>(nv_row + (nb * 16 + n) * 2);
      else nv[nb] = *reinterpret_cast<const uint32_t*>(nv_row + (nb * 16 + n) * 4);
    }
  }
  // evaluated where it is used, so that only those uses wait for the slot
  auto own_new = [&]() -> bool { return last_new && slot_new >= 0; };

  // q operand: head n of the group, zero beyond G (the row address is
  // clamped to a head of this group so that it always exists)
  uint4 qop[NX];
  {
    const int hq = h0 + min(n, G - 1);
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(s) * a.num_q_heads + hq) * D) * ELT;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const uint4 w = ld16(qb + (x * 4 + j4) * 16);
      qop[x] = n < G ? w : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const float c2 = a.scale * kLog2e;

  const char* kl = geo.k_base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  const char* vl = geo.v_base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  const int32_t* table = nullptr;
  int64_t first_block = 0;
  if (geo.paged) {
    table = a.tables + static_cast<int64_t>(s) * a.table_stride;
  } else {
    const int rid = a.req_ids ? a.req_ids[s] : s;
    first_block = static_cast<int64_t>(rid) * geo.blocks_per_seq;
  }
  // byte offset of tile (block of token t, kvh); t is clamped into the
  // context so that every address stays inside a block the sequence owns
  auto tile_of = [&](int t) -> int64_t {
    t = min(t, L - 1);
    const int64_t u = geo.paged ? static_cast<int64_t>(table[t / BS]) : first_block + t / BS;
    return (u * hkv + kvh) * TILE;
  };

  float m = -INFINITY;  // running max of head n (log2 units)
  float lsum = 0.0f;    // this lane's share of head n's weight sum
  floatx4_t acc[NN];    // acc[nb][i] = O[head 4*j4+i][dim nb*16+n]
#pragma unroll
  for (int nb = 0; nb < NN; ++nb) acc[nb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Wave-uniform block of chunk c (blocks of at least a chunk): a scalar load
  // of the table entry through the constant address space.  readfirstlane
  // keeps the index scalar even where the compiler cannot prove it uniform.
  auto block_of_chunk = [&](int c) -> int64_t {
    const int blk = __builtin_amdgcn_readfirstlane((c * kChunk) / BS);
    return geo.paged ? static_cast<int64_t>(__builtin_amdgcn_readfirstlane(
                           reinterpret_cast<const_i32_ptr>(reinterpret_cast<uintptr_t>(table))[blk]))
                     : first_block + blk;
  };
  // u: the chunk's block when BS >= kChunk (from block_of_chunk)
  auto load = [&](int c, int64_t u, uint4 (&kk)[NX], VOp (&vv)[NN]) {
    if constexpr (BS >= kChunk) {
      // the chunk lies in one block: a wave-uniform tile base plus a 32-bit
      // lane offset (rows past the context stay inside the tile)
      const int64_t tile = (u * hkv + kvh) * TILE;
      const char* kt = kl + tile;
      const char* vt = vl + tile;
      const int row0 = (c * kChunk) % BS;
      // the empty asm keeps each lane offset a 32-bit value inside the loop,
      // so that the loads use a scalar base plus a 32-bit vector offset
      // instead of a 64-bit vector address per lane
      uint32_t ko = static_cast<uint32_t>((j4 * BS + row0 + n) * 16);
      asm volatile("" : "+v"(ko));
#pragma unroll
      for (int x = 0; x < NX; ++x) kk[x] = kv16<NT>(kt + ko + x * 4 * BS * 16);
      uint32_t vo = static_cast<uint32_t>((n * BS + row0 + 4 * j4) * ELT);
      asm volatile("" : "+v"(vo));
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) vv[nb] = kv8<NT>(vt + vo + nb * 16 * BS * ELT);
        else vv[nb] = kv16<NT>(vt + vo + nb * 16 * BS * ELT);
      }
    } else {
      // blocks shorter than a chunk: each lane finds its own block
      const int tk = c * kChunk + n;
      const char* kt = kl + tile_of(tk) + (tk % BS) * 16;
#pragma unroll
      for (int x = 0; x < NX; ++x) kk[x] = kv16<NT>(kt + (x * 4 + j4) * BS * 16);
      int tv = c * kChunk + 4 * j4;
      tv = min(tv, ((L - 1) / 4) * 4);
      const char* vt = vl + tile_of(tv) + (tv % BS) * ELT;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) vv[nb] = kv8<NT>(vt + (nb * 16 + n) * BS * ELT);
        else vv[nb] = kv16<NT>(vt + (nb * 16 + n) * BS * ELT);
      }
    }
  };

  // the new token's K and V replace what the cache holds at position L-1
  // (selects only: a reference to a runtime-chosen component would send the
  // operand registers to scratch memory); the lanes holding them copy them
  // to LDS for the store after the loop
  auto patch_new = [&](int c, uint4 (&kk)[NX], VOp (&vv)[NN]) {
    const bool krow = c * kChunk + n == L - 1;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      kk[x].x = krow ? nk[x].x : kk[x].x;
      kk[x].y = krow ? nk[x].y : kk[x].y;
      kk[x].z = krow ? nk[x].z : kk[x].z;
      kk[x].w = krow ? nk[x].w : kk[x].w;
    }
    if (krow) {
#pragma unroll
      for (int x = 0; x < NX; ++x) sm_new[x * 4 + j4] = nk[x];
    }
    const int e = L - 1 - (c * kChunk + 4 * j4);
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) {
      const uint32_t h = nv[nb];
      if constexpr (KIND == kBF16) {
        const uint32_t x = vv[nb].x, y = vv[nb].y;
        vv[nb].x = e == 0 ? ((x & 0xFFFF0000u) | h) : (e == 1 ? ((x & 0x0000FFFFu) | (h << 16)) : x);
        vv[nb].y = e == 2 ? ((y & 0xFFFF0000u) | h) : (e == 3 ? ((y & 0x0000FFFFu) | (h << 16)) : y);
      } else {
        vv[nb].x = e == 0 ? h : vv[nb].x;
        vv[nb].y = e == 1 ? h : vv[nb].y;
        vv[nb].z = e == 2 ? h : vv[nb].z;
        vv[nb].w = e == 3 ? h : vv[nb].w;
      }
    }
    if (e >= 0 && e < 4) {
      char* nv_lds = reinterpret_cast<char*>(sm_new + kRowVec);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) reinterpret_cast<uint16_t*>(nv_lds)[nb * 16 + n] = static_cast<uint16_t>(nv[nb]);
        else reinterpret_cast<uint32_t*>(nv_lds)[nb * 16 + n] = nv[nb];
      }
    }
  };

  // one chunk: S = K q^T on the MFMA, online softmax, O += P V.  FIRST marks
  // a wave's first chunk, the only one that can be partly filled.
  auto process = [&](auto first, int c, uint4 (&kop)[NX], VOp (&vop)[NN]) {
    constexpr bool kFirst = decltype(first)::value;
    // S[token 4*j4+i][head n]
    floatx4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if constexpr (KIND == kBF16) {
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[x]),
                                                    __builtin_bit_cast(bf16x8_t, qop[x]), S, 0, 0, 0);
      } else {
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop[x].x), __uint_as_float(qop[x].x), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop[x].y), __uint_as_float(qop[x].y), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop[x].z), __uint_as_float(qop[x].z), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop[x].w), __uint_as_float(qop[x].w), S, 0, 0, 0);
      }
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = S[i] * c2;
    const int t0 = c * kChunk + 4 * j4;
    if (kFirst && (c + 1) * kChunk > L) {
      // last, partly filled chunk: rows past the context hold whatever the
      // cache held (possibly NaN or Inf patterns): zero weight and zero V
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + i >= L) sc[i] = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) {
          const uint32_t m0 = t0 + 0 < L ? 0x0000FFFFu : 0u, m1 = t0 + 1 < L ? 0xFFFF0000u : 0u;
          const uint32_t m2 = t0 + 2 < L ? 0x0000FFFFu : 0u, m3 = t0 + 3 < L ? 0xFFFF0000u : 0u;
          vop[nb].x &= (m0 | m1);
          vop[nb].y &= (m2 | m3);
        } else {
          if (t0 + 0 >= L) vop[nb].x = 0u;
          if (t0 + 1 >= L) vop[nb].y = 0u;
          if (t0 + 2 >= L) vop[nb].z = 0u;
          if (t0 + 3 >= L) vop[nb].w = 0u;
        }
      }
    }
    // online softmax for head n
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float mn = fmaxf(m, mx);
    // a wave's first chunk starts from m = -inf, acc = 0 and lsum = 0, so
    // there is nothing to rescale (and acc need not be live yet)
    const float alpha = kFirst ? 0.0f : fexp2(m - mn);
    m = mn;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fexp2(sc[i] - mn);
    if (!kFirst && __any(alpha != 1.0f)) {
      // rows of acc belong to heads 4*j4+i: fetch their factors
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j4 + i);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= ai[i];
    }
    if constexpr (KIND == kBF16) {
      // weight = high + low, both bf16; the sum is what the MFMA multiplies
      uint32_t hi01 = pack_bf16(p[0], p[1]), hi23 = pack_bf16(p[2], p[3]);
      const float h0f = bf16_lo(hi01), h1f = bf16_hi(hi01), h2f = bf16_lo(hi23), h3f = bf16_hi(hi23);
      const float r0 = p[0] - h0f, r1 = p[1] - h1f, r2 = p[2] - h2f, r3 = p[3] - h3f;
      uint32_t lo01 = pack_bf16(r0, r1), lo23 = pack_bf16(r2, r3);
      lsum = lsum * alpha + (((h0f + bf16_lo(lo01)) + (h1f + bf16_hi(lo01))) +
                             ((h2f + bf16_lo(lo23)) + (h3f + bf16_hi(lo23))));
      const short4_t phi = __builtin_bit_cast(short4_t, make_uint2(hi01, hi23));
      const short4_t plo = __builtin_bit_cast(short4_t, make_uint2(lo01, lo23));
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, __builtin_bit_cast(short4_t, vop[nb]),
                                                           acc[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, __builtin_bit_cast(short4_t, vop[nb]),
                                                           acc[nb], 0, 0, 0);
    } else {
      lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], __uint_as_float(vop[nb].x), acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], __uint_as_float(vop[nb].y), acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], __uint_as_float(vop[nb].z), acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], __uint_as_float(vop[nb].w), acc[nb], 0, 0, 0);
      }
    }
  };
  // The block of the next chunk is fetched one chunk ahead of its loads (an
  // index clamped into the partition rather than a branch).
  uint4 kbuf[NX];
  VOp vbuf[NN];
  int c = ce - 1 - wave;
  int64_t u_next = 0;
  if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c, cb));
  if (c >= cb) {
    const int64_t u = u_next;
    if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c - kWaves, cb));
    load(c, u, kbuf, vbuf);
    if (own_new()) patch_new(c, kbuf, vbuf);
    process(std::true_type{}, c, kbuf, vbuf);
    c -= kWaves;
  }
  while (c >= cb) {
    const int64_t u = u_next;
    if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c - kWaves, cb));
    load(c, u, kbuf, vbuf);
    process(std::false_type{}, c, kbuf, vbuf);
    c -= kWaves;
  }

  // weight sum of head n over the wave's tokens, then merge the waves:
  // LDS holds m[W][G], l[W][G], acc[W][G][D]
  extern __shared__ float lds[];
  float* sm_m = lds;
  float* sm_l = lds + kWaves * G;
  float* sm_acc = lds + 2 * kWaves * G;
  lsum += xor16(lsum);
  lsum += xor32(lsum);
  if (j4 == 0 && n < G) {
    sm_m[wave * G + n] = m;
    sm_l[wave * G + n] = lsum;
  }
#pragma unroll
  for (int nb = 0; nb < NN; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * j4 + i < G) sm_acc[(wave * G + 4 * j4 + i) * D + nb * 16 + n] = acc[nb][i];
  __syncthreads();
  const int64_t row0 = static_cast<int64_t>(s) * a.num_q_heads + h0;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, e = idx % D;
    float mx = sm_m[g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w * G + g]);
    float A = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fexp2(sm_m[w * G + g] - mx);
      A = fmaf(wt, sm_acc[(w * G + g) * D + e], A);
      Lt = fmaf(wt, sm_l[w * G + g], Lt);
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
  // the appended row into the cache: K as 16-byte pieces, V element by
  // element ([D][BS] tiles)
  if (own_new() && lane < kRowVec) {
    constexpr int VE = GG::VE;
    const int slot = slot_new;
    const int q = lane;
    const int64_t u = slot / BS;
    const int o = slot % BS;
    const int64_t tile = static_cast<int64_t>(a.layer) * geo.layer_bytes + (u * hkv + kvh) * TILE;
    *reinterpret_cast<uint4*>(geo.k_base + tile + (q * BS + o) * 16) = sm_new[q];
    const uint4 vw = sm_new[kRowVec + q];
    char* vt = geo.v_base + tile;
    const uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
    if constexpr (KIND == kBF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(vt + ((q * VE + 2 * e) * BS + o) * 2) = static_cast<uint16_t>(w[e] & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(vt + ((q * VE + 2 * e + 1) * BS + o) * 2) = static_cast<uint16_t>(w[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vt + ((q * VE + e) * BS + o) * 4) = w[e];
    }
  }
}

// Work plan of a launch split into partitions: plan[i] = {s * P + part, L_s}
// for the i-th (sequence, partition) with tokens to attend, {-1, 0} past the
// last.  Full partitions come first (in sequence order for up to 1024
// sequences), then every context's last partition, longest first
// (kPlanBuckets length classes; the order within a class varies between
// runs, which changes no result: each partition is computed on its own and
// merged in partition order).  Shared
// prefixes (seq_shared) are left out.  The partition kernel's grid then ends
// on its shortest workgroups, and the items without work (contexts shorter
// than the longest) come after all others instead of among them.  One
// workgroup.
constexpr int kPlanThreads = 1024;
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
// kMergeWaves rows per workgroup.  Lane l holds the running max and weight sum
// of partition p0 + l (64 partitions a round) and D / 64 output dims; a row's
// loads are all issued before its arithmetic.  The sums run over p in order,
// as fma(w_p, acc_p, .) and fma(w_p, l_p, .).
template <int D>
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
  if (ps > 0) {
    float mx = -INFINITY;
    for (int p0 = 0; p0 < ps; p0 += kWave)
      if (p0 + lane < ps) mx = fmaxf(mx, ml[2 * (p0 + lane)]);
#pragma unroll
    for (int x = kWave / 2; x >= 1; x /= 2) mx = fmaxf(mx, __shfl_xor(mx, x));
    float Lt = 0.0f;
    for (int p0 = 0; p0 < ps; p0 += kWave) {
      float wl = 0.0f, ll = 0.0f;
      if (p0 + lane < ps) {
        wl = fexp2(ml[2 * (p0 + lane)] - mx);
        ll = ml[2 * (p0 + lane) + 1];
      }
      const int n = min(kWave, ps - p0);
      const float* ap = accp + static_cast<int64_t>(p0) * D;
#pragma unroll 8
      for (int k = 0; k < n; ++k) {
        const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k));
        const float lk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ll), k));
#pragma unroll
        for (int e = 0; e < E; ++e) A[e] = fmaf(wt, ap[k * D + e], A[e]);
        Lt = fmaf(wt, lk, Lt);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) A[e] = A[e] / Lt;
  }
  if constexpr (E == 2) {
    *reinterpret_cast<float2*>(o) = make_float2(A[0], A[1]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = A[e];
  }
}

// ---------------------------------------------------------------------------
// append and copy-on-write copies
// ---------------------------------------------------------------------------
// One thread per (token, KV head, 16-byte chunk of the row): the K chunk is
// stored whole, the V chunk's elements go to their dims' rows of the V tile.
__global__ __launch_bounds__(256) void append_kv_kernel(CacheGeom g, int32_t layer,
                                                        const uint4* __restrict__ k,
                                                        const uint4* __restrict__ v,
                                                        const int32_t* __restrict__ slots,
                                                        int32_t n) {
  const int ve = 16 / g.elt;
  const int chunks = g.head_dim / ve;
  const int per_tok = g.num_kv_heads * chunks;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n) * per_tok) return;
  const int i = static_cast<int>(idx / per_tok);
  const int rem = static_cast<int>(idx % per_tok);
  const int h = rem / chunks, q = rem % chunks;
  const int slot = slots[i];
  if (slot < 0) return;
  const int64_t u = slot / g.block_size;
  const int o = slot % g.block_size;
  const int64_t tile = static_cast<int64_t>(layer) * g.layer_bytes +
                       (u * g.num_kv_heads + h) * (static_cast<int64_t>(g.head_dim) * g.block_size * g.elt);
  *reinterpret_cast<uint4*>(g.k_base + tile + (static_cast<int64_t>(q) * g.block_size + o) * 16) = k[idx];
  const uint4 w = v[idx];
  char* vt = g.v_base + tile;
  const int d0 = q * ve;
  if (g.elt == 2) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint16_t*>(vt + ((d0 + 2 * e) * g.block_size + o) * 2) =
          static_cast<uint16_t>(ws[e] & 0xFFFFu);
      *reinterpret_cast<uint16_t*>(vt + ((d0 + 2 * e + 1) * g.block_size + o) * 2) =
          static_cast<uint16_t>(ws[e] >> 16);
    }
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint32_t*>(vt + ((d0 + e) * g.block_size + o) * 4) = ws[e];
  }
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

template <int KIND, int D, int BS, int W>
hipError_t launch_decode_w(const CacheGeom& g, const DecodeArgs& a, hipStream_t st) {
  const int64_t nwork = static_cast<int64_t>(a.num_seqs) * g.num_kv_heads * a.num_partitions;
  const int G = a.num_q_heads / g.num_kv_heads;
  if (a.streaming)
    hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, W, true>), dim3(static_cast<uint32_t>(nwork)),
                       dim3(W * kWave), merge_lds_bytes(W, G, D), st, g, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<KIND, D, BS, W, false>), dim3(static_cast<uint32_t>(nwork)),
                       dim3(W * kWave), merge_lds_bytes(W, G, D), st, g, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const DecodeArgs& a, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(static_cast<uint32_t>((rows + kMergeWaves - 1) / kMergeWaves)),
                     dim3(kMergeWaves * kWave), 0, st, a);
  return hipGetLastError();
}

template <int KIND, int D, int BS>
hipError_t launch_decode_t(const CacheGeom& g, const DecodeArgs& a, hipStream_t st) {
  const int G = a.num_q_heads / g.num_kv_heads;
  if (a.waves == 8 && merge_lds_bytes(8, G, D) <= kMaxMergeLds)
    return launch_decode_w<KIND, D, BS, 8>(g, a, st);
  return launch_decode_w<KIND, D, BS, 4>(g, a, st);
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
  if (a.num_q_heads / g.num_kv_heads > kMaxGroup || (g.head_dim != 128 && g.head_dim != 64)) {
    *supported = false;
    return hipSuccess;
  }
  DecodeArgs ap = a;
  // Split launches run from a plan (decode_plan_kernel), except after a
  // shared-prefix pass: there every context has one private partition left,
  // and the plan's launch costs more (measured) than the skipped partitions.
  if (a.num_partitions > 1 && a.seq_shared == nullptr) {
    // the plan follows the partials in the workspace
    int2* plan = reinterpret_cast<int2*>(a.ws + static_cast<int64_t>(a.num_seqs) * a.num_q_heads *
                                                    a.num_partitions * (g.head_dim + 2));
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, plan);
    hipError_t ep = hipGetLastError();
    if (ep != hipSuccess) return ep;
    ap.plan = plan;
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
