// The decode partition kernel's body: attention of one query token per
// request over K/V held in fixed blocks reached through a block table
// ("Running Out of Cache", paging paragraph and Terms), or over a per-request
// sub-tensor at reqId x S ("Leveraging Low-Level CUDA APIs for vAttention's
// Dynamic Memory", 5.2.3), for one context partition of one (sequence, KV
// head).  kernels.hip launches it alone; the shared-prefix launch in
// decode_shared.hip runs it for the private partitions beside the shared
// pass.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "decode_common.hpp"
#include "kernels.hpp"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// decode: one workgroup per (sequence, KV head, partition)
// ---------------------------------------------------------------------------
// bf16 caches with blocks of at least a chunk fit 128 VGPRs, i.e. four waves
// per SIMD (the occupancy the HBM stream needs); the others would spill.
template <int KIND, int BS>
constexpr int decode_min_waves_per_eu() { return KIND == kBF16 && BS >= kChunk ? 4 : 1; }
// The two-chunk pipeline (PIPE) keeps a second chunk's K/V operands in
// registers; it runs only on grids of at most one wave per SIMD, so it may
// take up to 256 VGPRs.  The balanced start (BAL) holds a second operand set
// in the first step only; it runs on grids of at most two waves per SIMD.
// Both exist for bf16 caches whose blocks hold whole chunks.
template <int KIND, int BS, bool PIPE, bool BAL = false>
constexpr int decode_waves_per_eu() { return PIPE || BAL ? 2 : decode_min_waves_per_eu<KIND, BS>(); }
template <int KIND, int BS>
constexpr bool decode_pipe_ok() { return KIND == kBF16 && BS >= kChunk; }
// LDS bytes of the wave merge: per wave, G maxima, G sums and G x D partial
// outputs.
__host__ __device__ constexpr int merge_lds_bytes(int waves, int G, int D) {
  return waves * G * (D + 2) * 4;
}
// LDS bytes after the merge area that a fused append uses: with blocks of
// at least a chunk it stages its tail chunk there (the chunk's V tile rows,
// D x 16 tokens, the two K rows that share the new row's 32-byte sectors, and
// the slot); with shorter blocks it keeps the new row (K pieces, V pieces)
// for the store after the loop.
__host__ __device__ constexpr int append_lds_bytes(int D, int elt, int bs) {
  return bs >= 16 ? D * 16 * elt + 2 * D * elt + 16 : 2 * D * elt;
}

// The body of decode_partition_kernel for workgroup `bid` of `nblocks`, with
// `lds` the launch's dynamic LDS (at least merge_lds_bytes(W, G, D) bytes):
// also run by the workgroups of the shared-prefix launch that do the
// private partitions.  PIPE: each wave keeps the loads of its next chunk in
// flight while it computes the current one.  BAL: the waves that hold one
// chunk more than the others load their first two chunks together.
template <int KIND, int D, int BS, int W, bool NT, bool PIPE = false, bool BAL = false, bool PAIRED = false>
__device__ __forceinline__ void decode_partition_body(const CacheGeom& geo, const DecodeArgs& a, int bid,
                                                      int nblocks, float* lds) {
  using GG = Geo<KIND, D, BS>;
  constexpr int NX = GG::NX, NN = GG::NN, CH = GG::CH, SUBPAIR = GG::SUBPAIR, PAIR = GG::PAIR, ELT = GG::ELT;
  constexpr int kWaves = W;
  constexpr int kThreads = W * kWave;
  // V operand per lane per output tile: 4 consecutive tokens of one dim
  using VOp = typename std::conditional<KIND == kBF16, uint2, uint4>::type;

  const int P = a.num_partitions;
  const int hkv = geo.num_kv_heads;
  const int G = a.num_q_heads / hkv;
  // With a plan (large split launches), workgroup i takes the KV head i % hkv
  // of plan item i / hkv; the items with work fill the front of the grid,
  // longest first, and the grid's tail exits at once.  Without one, work
  // items are (r, sequence, KV head), r-major, with r a partition's place
  // counted from the end of its context: with one partition per context
  // that is each context's only one; in a small split launch r runs
  // downwards, so that each context's last, partly filled partition comes
  // last; after a shared-prefix pass it runs upwards, so that the private
  // partitions (the last ones) come first and the shared ones, which exit at
  // once, after them.
  // PAIRED: the workgroup runs two work items, one per W waves, each with
  // its own LDS; every wave then passes exactly one barrier, the merge's or
  // (leaving early) the one in leave()
  const int tid = PAIRED ? static_cast<int>(threadIdx.x) % kThreads : static_cast<int>(threadIdx.x);
  auto leave = [] {
    if constexpr (PAIRED) __syncthreads();
  };
  // A balanced-start grid is at most two workgroups per CU, all resident
  // from the start; the second one on a CU (ids from kComputeUnits on, as the
  // dispatcher deals them) loses the SIMDs' issue arbitration to the older
  // first one and finished about 1.3 us later on the Llama-3-8B batch-64
  // layer (per-wave clocks).  Its waves issue at a higher priority instead.
  if constexpr (BAL) {
    if (bid >= kComputeUnits) __builtin_amdgcn_s_setprio(1);
  }
  int s, kvh, part, L;
  if (a.plan != nullptr) {
    const int2 it = a.plan[bid / hkv];
    if (it.x < 0 || it.x >= a.num_seqs * P) return leave();
    s = it.x / P;
    part = it.x % P;
    kvh = bid % hkv;
    L = min(max(it.y, 0), a.max_context);
  } else {
    const int work = work_item(bid, nblocks, !NT);
    const int pairs = a.num_seqs * hkv;
    const int r = a.seq_shared != nullptr ? work / pairs : P - 1 - work / pairs;
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
      return leave();
    }
  }
  const int h0 = kvh * G;
  const int nch = (L + kChunk - 1) / kChunk;
  const int cb = part * a.partition_chunks;
  const int ce = min(nch, cb + a.partition_chunks);
  if (a.seq_shared != nullptr && cb * kChunk < a.seq_shared[s]) return leave();  // the shared pass's

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
  // first chunk, where selects put it into the operand registers; the
  // stores into the cache come after the loop, from LDS.  (Stores issued
  // during the loop, where they interleave with the reads, cost more.)
  // The row and the slot are loaded whatever the slot says: only their use
  // waits for the slot (a slot < 0 appends nothing and the cache is read as
  // it is), so no load of the workgroup's start waits on another.
  constexpr int kRowVec = D * ELT / 16;  // 16-byte pieces of one row
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
  // With blocks of at least a chunk the new row is stored as whole 32-byte
  // sectors: the tail chunk's V rows and the K row sharing each of the new
  // row's K sectors, staged in LDS past the merge area as they were loaded
  // (plus the new row), are written back after the loop, so every other
  // byte goes back unchanged.  Partial-sector stores of the row alone cost
  // 1.9 us of the 47 us launch on the Llama-3-8B batch-64 layer.
  constexpr bool kWholeSectors = BS >= kChunk;
  const bool wg_appends = a.new_k != nullptr && ce == nch;   // the same in every wave
  char* stage = reinterpret_cast<char*>(lds) + merge_lds_bytes(kWaves, G, D);
  char* stage_v = stage;                                    // [D][16] elements
  char* stage_k = stage + D * kChunk * ELT;                 // [2][D] elements
  int* stage_slot = reinterpret_cast<int*>(stage_k + 2 * D * ELT);
  // blocks shorter than a chunk: the new row's K pieces, then its V pieces
  uint4* sm_new = reinterpret_cast<uint4*>(stage);

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

  // K tiles of the layer; each V tile follows its K tile
  const char* kl = geo.base + static_cast<int64_t>(a.layer) * geo.layer_bytes;
  const char* vl = kl + CH;
  const int32_t* table = nullptr;
  int64_t first_block = 0;
  if (geo.paged) {
    table = a.tables + static_cast<int64_t>(s) * a.table_stride;
  } else {
    const int rid = a.req_ids ? a.req_ids[s] : s;
    first_block = static_cast<int64_t>(rid) * geo.blocks_per_seq;
  }

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
      // the chunk is one tile pair of its block: a wave-uniform pair base
      // plus a 32-bit lane offset (rows past the context stay inside it)
      const int64_t tile = (u * hkv + kvh) * PAIR + ((c * kChunk) % BS / kChunk) * SUBPAIR;
      const char* kt = kl + tile;
      const char* vt = vl + tile;
      // the empty asm keeps each lane offset a 32-bit value inside the loop,
      // so that the loads use a scalar base plus a 32-bit vector offset
      // instead of a 64-bit vector address per lane
      uint32_t ko = static_cast<uint32_t>((j4 * kChunk + n) * 16);
      asm volatile("" : "+v"(ko));
#pragma unroll
      for (int x = 0; x < NX; ++x) kk[x] = kv16<NT>(kt + ko + x * 4 * kChunk * 16);
      uint32_t vo = static_cast<uint32_t>((n * kChunk + 4 * j4) * ELT);
      asm volatile("" : "+v"(vo));
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) vv[nb] = kv8<NT>(vt + vo + nb * 16 * kChunk * ELT);
        else vv[nb] = kv16<NT>(vt + vo + nb * 16 * kChunk * ELT);
      }
    } else {
      // blocks shorter than a chunk: the chunk spans blocks j0 and j0 + 1
      // (the second clamped into the context); both table entries are
      // wave-uniform scalar loads and each lane takes its token's (a table
      // entry per lane would be a dependent vector load)
      const int j0 = (c * kChunk) / BS;
      const int j1 = min(j0 + 1, (L - 1) / BS);
      auto entry = [&](int j) -> int64_t {
        return geo.paged ? static_cast<int64_t>(__builtin_amdgcn_readfirstlane(
                               reinterpret_cast<const_i32_ptr>(reinterpret_cast<uintptr_t>(table))[j]))
                         : first_block + j;
      };
      const int64_t p0 = (entry(j0) * hkv + kvh) * PAIR, p1 = (entry(j1) * hkv + kvh) * PAIR;
      auto pair_of = [&](int t) -> int64_t { return min(t, L - 1) / BS == j0 ? p0 : p1; };
      const int tk = c * kChunk + n;
      const char* kt = kl + pair_of(tk) + (tk % BS) * 16;
#pragma unroll
      for (int x = 0; x < NX; ++x) kk[x] = kv16<NT>(kt + (x * 4 + j4) * BS * 16);
      int tv = c * kChunk + 4 * j4;
      tv = min(tv, ((L - 1) / 4) * 4);
      const char* vt = vl + pair_of(tv) + (tv % BS) * ELT;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        if constexpr (KIND == kBF16) vv[nb] = kv8<NT>(vt + (nb * 16 + n) * BS * ELT);
        else vv[nb] = kv16<NT>(vt + (nb * 16 + n) * BS * ELT);
      }
    }
    // every load of the chunk issues before anything that waits for one:
    // left to itself the scheduler slots the first score MFMAs (and their
    // waits) between the K and the V loads, so V leaves for memory only
    // after K has come back
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
    if constexpr (!kWholeSectors) {
      if (krow) {
#pragma unroll
        for (int x = 0; x < NX; ++x) sm_new[x * 4 + j4] = nk[x];
      }
    } else {
      // K rows o and o ^ 1 of the chunk (o = the new row), patched
      if ((n >> 1) == (((L - 1) % kChunk) >> 1)) {
#pragma unroll
        for (int x = 0; x < NX; ++x)
          *reinterpret_cast<uint4*>(stage_k + ((n & 1) * D * ELT) + (x * 4 + j4) * 16) = kk[x];
      }
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
    if constexpr (kWholeSectors) {
      // the chunk's V as loaded, with the new row: tokens 4*j4 .. 4*j4+3 of
      // dim nb*16+n
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) *reinterpret_cast<VOp*>(stage_v + ((nb * 16 + n) * kChunk + 4 * j4) * ELT) = vv[nb];
    } else if (e >= 0 && e < 4) {
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
  uint4 kbuf[NX];
  VOp vbuf[NN];
  int c = ce - 1 - wave;
  if constexpr (PIPE) {
    static_assert(decode_pipe_ok<KIND, BS>(), "the pipeline needs whole chunks per block");
    // Two operand sets, A (kbuf, vbuf) and B (kb2, vb2), used in turn: the
    // loads of chunk c - W are issued before chunk c is computed.  Every
    // branch below is taken after the loads it depends on were issued on all
    // paths into it, so the wait before a chunk's arithmetic covers that
    // chunk's loads and not the next ones.
    uint4 kb2[NX];
    VOp vb2[NN];
    if (c >= cb) {
      load(c, block_of_chunk(c), kbuf, vbuf);
      if (c - kWaves >= cb) {
        load(c - kWaves, block_of_chunk(c - kWaves), kb2, vb2);
        if (kWholeSectors && last_new && lane == 0) *stage_slot = slot_new;
        if (own_new()) patch_new(c, kbuf, vbuf);
        process(std::true_type{}, c, kbuf, vbuf);
        c -= kWaves;
        // here chunk c >= cb is in flight in B
        while (true) {
          if (c - kWaves < cb) { process(std::false_type{}, c, kb2, vb2); break; }
          load(c - kWaves, block_of_chunk(c - kWaves), kbuf, vbuf);
          process(std::false_type{}, c, kb2, vb2);
          c -= kWaves;
          if (c - kWaves < cb) { process(std::false_type{}, c, kbuf, vbuf); break; }
          load(c - kWaves, block_of_chunk(c - kWaves), kb2, vb2);
          process(std::false_type{}, c, kbuf, vbuf);
          c -= kWaves;
        }
      } else {
        if (kWholeSectors && last_new && lane == 0) *stage_slot = slot_new;
        if (own_new()) patch_new(c, kbuf, vbuf);
        process(std::true_type{}, c, kbuf, vbuf);
      }
    }
  } else {
    // The block of the next chunk is fetched one chunk ahead of its loads (an
    // index clamped into the partition rather than a branch).
    int64_t u_next = 0;
    if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c, cb));
    // Balanced start (BAL): when the partition's n chunks are not a multiple
    // of W, waves w < n % W hold one chunk more than the others.  They load
    // their first two chunks together, so that no wave takes an extra HBM
    // round trip while the others have finished (Llama-3-8B batch-64 layer:
    // 46.5 -> 46.0 us; Yi-34B share 47.3 -> 46.5 us).
    const int n_ch = ce - cb;
    const bool extra = BAL && BS >= kChunk && wave < n_ch % kWaves && c - kWaves >= cb;
    if (c >= cb) {
      const int64_t u = u_next;
      if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c - kWaves, cb));
      load(c, u, kbuf, vbuf);
      if (kWholeSectors && last_new && lane == 0) *stage_slot = slot_new;
      if (BAL && extra) {
        uint4 kb2[NX];
        VOp vb2[NN];
        const int64_t u2 = u_next;
        if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c - 2 * kWaves, cb));
        load(c - kWaves, u2, kb2, vb2);
        if (own_new()) patch_new(c, kbuf, vbuf);
        process(std::true_type{}, c, kbuf, vbuf);
        process(std::false_type{}, c - kWaves, kb2, vb2);
        c -= 2 * kWaves;
      } else {
        if (own_new()) patch_new(c, kbuf, vbuf);
        process(std::true_type{}, c, kbuf, vbuf);
        c -= kWaves;
      }
    }
    while (c >= cb) {
      const int64_t u = u_next;
      if constexpr (BS >= kChunk) u_next = block_of_chunk(max(c - kWaves, cb));
      load(c, u, kbuf, vbuf);
      process(std::false_type{}, c, kbuf, vbuf);
      c -= kWaves;
    }
  }

  // weight sum of head n over the wave's tokens, then merge the waves:
  // LDS holds m[W][G], l[W][G], acc[W][G][D]
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
      __builtin_nontemporal_store(A / Lt, &a.out[(row0 + g) * D + e]);
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
  // Where no split-K partial follows them (one partition per context) the
  // appended row's stores and the output are the launch's last traffic and
  // go out non-temporal (measurements at st16 below)
  const bool nt_end = BAL || PAIRED || P == 1;
  if constexpr (kWholeSectors) {
    // whole sectors from the staged chunk, by every thread: the chunk's D V
    // rows (16 tokens each) and K rows o & ~1, o | 1 of every 16-byte piece
    if (wg_appends) {
      const int slot = *stage_slot;
      if (slot >= 0) {
        const int64_t u = slot / BS;
        const int o = slot % BS;                 // row in the block
        const int oc = o % kChunk;                // row in the chunk (its tile pair)
        char* kt = geo.base + static_cast<int64_t>(a.layer) * geo.layer_bytes + (u * hkv + kvh) * PAIR +
                   (o / kChunk) * SUBPAIR;
        char* vt = kt + CH;
        constexpr int kVUnits = D * kChunk * ELT / 16;   // 16-byte units of the chunk's V
        // Non-temporal where no split-K partial follows: Llama-3-8B batch-64
        // layer 45.49 -> 44.75 us, Yi-34B share 46.57 -> 45.73 us, Yi-6B
        // shared-prefix workload read per sample 133.9 -> 132.2 us, batch
        // 256 x 512 tokens 100.7 -> 99.3 us; the shared-prefix launch's
        // private items (PAIRED) too: Yi-6B step 82.15 -> 80.74 us.  On the
        // split ragged mix the same change cost 1.2 us (233.1 against 232.0
        // us), so split launches keep ordinary stores.
        auto st16 = [nt_end](char* dst, const char* src) {
          if (nt_end)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(src), reinterpret_cast<u32x4_t*>(dst));
          else
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        };
        for (int t = tid; t < kVUnits; t += kThreads) st16(vt + t * 16, stage_v + t * 16);
        for (int t = tid; t < 2 * kRowVec; t += kThreads) {
          const int r = t / kRowVec, q = t % kRowVec;   // row (oc & ~1) + r, piece q
          st16(kt + (q * kChunk + (oc & ~1) + r) * 16, stage_k + r * D * ELT + q * 16);
        }
      }
    }
  }
  // the appended row into the cache: K as 16-byte pieces, V element by
  // element ([D][BS] tiles)
  if (!kWholeSectors && own_new() && lane < kRowVec) {
    constexpr int VE = GG::VE;
    const int slot = slot_new;
    const int q = lane;
    const int64_t u = slot / BS;
    const int o = slot % BS;
    char* kt = geo.base + static_cast<int64_t>(a.layer) * geo.layer_bytes + (u * hkv + kvh) * PAIR;
    // non-temporal on one-partition launches, as above (8-token blocks:
    // Llama-3-8B batch-64 layer 46.32 -> 45.50 us, Yi-34B share 46.98 ->
    // 46.47 us)
    const uint4 kw = sm_new[q];
    char* kd = kt + (q * BS + o) * 16;
    if (nt_end) __builtin_nontemporal_store(u32x4_t{kw.x, kw.y, kw.z, kw.w}, reinterpret_cast<u32x4_t*>(kd));
    else *reinterpret_cast<uint4*>(kd) = kw;
    const uint4 vw = sm_new[kRowVec + q];
    char* vt = kt + CH;
    const uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
    if constexpr (KIND == kBF16) {
      auto st2 = [nt_end](char* dst, uint16_t x) {
        if (nt_end) __builtin_nontemporal_store(x, reinterpret_cast<uint16_t*>(dst));
        else *reinterpret_cast<uint16_t*>(dst) = x;
      };
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st2(vt + ((q * VE + 2 * e) * BS + o) * 2, static_cast<uint16_t>(w[e] & 0xFFFFu));
        st2(vt + ((q * VE + 2 * e + 1) * BS + o) * 2, static_cast<uint16_t>(w[e] >> 16));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vt + ((q * VE + e) * BS + o) * 4) = w[e];
    }
  }
}

}  // namespace
}  // namespace pa
