// Launchers of the HIP kernels behind libpa.so (internal; the public ABI is
// include/pa.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

enum Kind : int { kF32 = 0, kBF16 = 1 };

// Waves per workgroup of the decode partition kernel.
constexpr int kDecodeWaves = 4;

// Cache geometry.  One array holds K and V of every layer.  Per layer it is
// an array of (block, KV head) regions of 2*tile_bytes each.  A region holds
// block_size / sub tile pairs, sub = min(block_size, 16) token rows each: the
// K tile, then the V tile of the same rows, so that a 16-token chunk is one
// contiguous run (2 x 4 KiB for bf16, head_dim 128):
//   K tile [head_dim/VE][sub][VE]  (16-byte chunks, VE = 16/elt)
//   V tile [head_dim][sub]
// Region (u, h) of layer l starts at l*layer_bytes + (u*num_kv_heads + h) *
// 2*tile_bytes from the base; row o's pair o / sub pairs further on.  Paged:
// u is the physical block.  Contiguous: request r owns blocks
// r*blocks_per_seq .. r*blocks_per_seq + blocks_per_seq - 1.  A slot is
// u*block_size + row.
struct CacheGeom {
  char* base = nullptr;        // layer 0, block 0, head 0, K tile
  int64_t layer_bytes = 0;     // bytes of one layer (K and V)
  int64_t tile_bytes = 0;      // K (or V) bytes of one (block, head): head_dim * block_size * elt
  int32_t num_layers = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t elt = 0;             // bytes per element
  int32_t block_size = 0;
  int32_t blocks_per_seq = 0;  // contiguous: max_seq_len / block_size
  int32_t paged = 1;
};

hipError_t launch_append(const CacheGeom& g, int32_t layer, const void* k, const void* v,
                         const int32_t* slots, int32_t n, hipStream_t stream);

hipError_t launch_copy_blocks(const CacheGeom& g, const int32_t* pairs, int32_t n,
                              hipStream_t stream);

// Swap image <-> blocks: blocks[j] (host array, n ids) in every layer, to or
// from image[layer][j][num_kv_heads][K|V][tile] (device-addressable): each
// block's tile pairs of a layer, as the cache holds them.
hipError_t launch_swap(const CacheGeom& g, const int32_t* blocks, int32_t n, char* image,
                       bool to_image, hipStream_t stream);

struct DecodeArgs {
  const void* q = nullptr;           // [B][Hq][D]
  const int32_t* tables = nullptr;   // paged: [B][stride]
  const int32_t* req_ids = nullptr;  // contiguous: [B] or null
  const int32_t* lens = nullptr;     // [B]
  float* out = nullptr;              // [B][Hq][D]
  float* ws = nullptr;               // partials when num_partitions > 1
  int32_t layer = 0;
  int32_t num_seqs = 0;
  int32_t num_q_heads = 0;
  int32_t table_stride = 0;
  int32_t partition_chunks = 0;      // 16-token chunks per partition
  int32_t num_partitions = 1;
  int32_t max_context = 0;           // no context is longer (tables hold its blocks)
  // fused append (pa_append_decode): token L_s - 1 of sequence s is
  // new_k[s] / new_v[s] ([B][Hkv][D]), stored to slot new_slots[s] (< 0: none)
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  const int32_t* new_slots = nullptr;
  int32_t streaming = 1;             // non-temporal K/V loads (no block is shared)
  float scale = 1.0f;
  // shared-prefix decode: the first seq_shared[s] tokens of sequence s (whole
  // partitions) are attended by decode_shared_kernel; the partition kernel
  // skips them.  Null: none.
  const int32_t* seq_shared = nullptr;
  // work plan of a split launch (decode_plan_kernel's output in the
  // workspace): item i = {s * num_partitions + partition, L_s}, {-1, 0} past
  // the last.  Null: the grid enumerates every (partition, sequence, head).
  // Items outside [0, num_seqs * num_partitions) are skipped and lengths
  // clamped to [0, max_context], so a plan made for other lengths gives
  // wrong results but no access outside the caller's arrays.
  const int2* plan = nullptr;
};

// Groups of sequences whose contexts start with the same blocks
// (pa_decode_shared): group i is sequences groups[2i] .. groups[2i] +
// groups[2i+1] - 1 of the batch, all with seq_shared[groups[2i]] shared tokens.
struct SharedArgs {
  const int32_t* groups = nullptr;   // [num_groups][2]: first sequence, members
  int32_t num_groups = 0;
  int32_t col_blocks = 1;            // workgroups per (group, KV head, partition): 64 query columns each
  int32_t shared_parts = 0;          // partitions of the longest shared prefix
  int32_t n_shared = 0;              // shared-pass workgroups: groups x KV heads x col_blocks x shared_parts
  // set by the launch: partition work items (sequences x KV heads x
  // partitions, two per workgroup) and the LDS bytes of each one
  int32_t n_private = 0;
  int32_t private_lds = 0;
};

// Whether a launch with these arguments runs from a work plan: split
// launches of at least two rounds of resident workgroups, without shared
// prefixes.
bool decode_uses_plan(const CacheGeom& g, const DecodeArgs& a);

// The work plan of such a launch, into its place in the workspace (after the
// partials); nothing for other launches.
hipError_t launch_decode_plan(const CacheGeom& g, const DecodeArgs& a, hipStream_t stream);

// The partition kernel and, with several partitions, the merge; the plan
// first where the launch uses one, unless plan_made (a launch_decode_plan for
// the same lengths, sizes and workspace ran before it on the stream).
// *supported is set to false (and nothing is launched) when no kernel exists
// for the shape.
hipError_t launch_decode(const CacheGeom& g, int kind, const DecodeArgs& a, bool* supported,
                         hipStream_t stream, bool plan_made = false);

// The merge of a split launch's partials (nothing when unsplit).
hipError_t launch_merge(const CacheGeom& g, const DecodeArgs& a, hipStream_t stream);

// Shared-prefix decode in one launch: the partials of every group's shared
// partitions, for all its members' query heads, and beside them the private
// partitions (a.seq_shared and the split-K workspace are set); the merge
// (launch_merge) must follow.
hipError_t launch_decode_shared(const CacheGeom& g, int kind, const DecodeArgs& a,
                                const SharedArgs& sh, bool* supported, hipStream_t stream);

// Device scratch of the allocation-free decode entry point
// (pa_append_decode_noalloc): a file-scope __device__ array in kernels.hip,
// one copy per GPU, held until the process ends.
constexpr size_t kStaticScratchBytes = static_cast<size_t>(64) << 20;

// Device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept.
hipError_t static_scratch(void** ptr);

// Bytes of decode partials for these sizes, then the work plan (one int2
// per (sequence, partition)).
inline size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                     int32_t num_partitions) {
  if (num_partitions <= 1) return 0;
  return static_cast<size_t>(num_seqs) * num_q_heads * num_partitions *
             (static_cast<size_t>(head_dim) + 2) * sizeof(float) +
         static_cast<size_t>(num_seqs) * num_partitions * 2 * sizeof(int32_t);
}

}  // namespace pa
