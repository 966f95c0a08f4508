// Device helpers shared by the decode kernels (kernels.hip, decode_shared.hip):
// wave constants, vector types, cache-read flavours, bf16 packing, and the
// per-shape constants of the tile layout (per (block, head), tile pairs of
// up to 16 token rows: K [D/VE][rows][VE], then V [D][rows]).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kComputeUnits = 256;  // MI355X: 8 XCDs x 32 CUs
constexpr int kChunk = 16;        // tokens per MFMA tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Workgroups of a launch are dealt to the 8 XCDs round-robin by id.  With
// shared blocks (samples of one prompt), give each XCD one contiguous range
// of work items so that the sharers meet in the same L2.  Without sharing,
// keep the round-robin order: the KV heads of one sequence then spread over
// all XCDs, which balances ragged batches (measured on MI355X: 4% faster on a
// ragged mix, 2% slower with shared prompts).
__device__ __forceinline__ int work_item(int bid, int n, bool group) {
  if (!group) return bid;
  constexpr int kXcd = 8;
  const int q = n / kXcd, rem = n % kXcd;
  const int x = bid % kXcd, local = bid / kXcd;
  return (x < rem) ? x * (q + 1) + local : rem * (q + 1) + (x - rem) * q + local;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// lane ^ 16 and lane ^ 32
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (16 << 10)));
}
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

// K/V cache reads.  When no block is shared, every byte is read once per
// decode and the loads are marked non-temporal (streamed past the caches'
// retention); shared blocks (several samples of one prompt) are read with
// ordinary loads so that the repeats hit in L2 / Infinity Cache.
// Read-only during a launch: a uniform read through the constant address
// space is always a scalar (SMEM) load, whatever else the kernel stores.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint4 kv16(const char* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return ld16(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 kv8(const char* p) {
  if constexpr (NT) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return ld8(p);
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int KIND, int D, int BS>
struct Geo {
  static constexpr int ELT = KIND == kBF16 ? 2 : 4;
  static constexpr int VE = 16 / ELT;          // elements per 16-byte K chunk
  static constexpr int NX = D / (4 * VE);      // 16-byte K loads per lane per chunk
  static constexpr int NN = D / 16;            // 16-column output tiles
  // A (block, head) holds BS / SUB tile pairs of SUB = min(BS, 16) token
  // rows each: the K tile [D/VE][SUB][VE], then the V tile [D][SUB].  With
  // blocks of 16 or 32 every 16-token chunk is one pair, one contiguous run.
  static constexpr int SUB = BS < kChunk ? BS : kChunk;
  static constexpr int CH = D * SUB * ELT;     // bytes of one K (or V) tile of a pair
  static constexpr int SUBPAIR = 2 * CH;       // one pair: K tile, then V tile
  static constexpr int PAIR = D * BS * ELT * 2;  // all pairs of a (block, head)
};

}  // namespace
}  // namespace pa
