/* A C caller of libpa.so: one decode iteration of a small paged cache through
 * the C ABI alone (include/pa.h), with device memory from the HIP runtime and
 * no Python in between.  tests/test_gpu_c_abi.py writes the inputs, runs this
 * program and checks its outputs against the oracle.
 *
 *   c_abi_decode <input file> <output file>
 *
 * Input (little-endian): int32 B, Hq, Hkv, D, BS, NB, layers, max_seq_len,
 * partition_tokens; int32 lens[B] (each >= 1: the decode step appends token
 * L-1); int32 free_order[NB]; float32 q[layers][B][Hq][D]; float32
 * k[layers][sum L][Hkv][D] and v likewise (the logical rows, sequence after
 * sequence).  The cache is fp32 and paged.
 *
 * The program admits B requests, reserves and appends every token but the
 * last (pa_reserve, pa_append_kv), reserves the step's token, and decodes
 * layer 0 with pa_append_decode and layer 1 with pa_decode_plan followed by
 * pa_append_decode_planned.
 *
 * Output: int32 planned (what pa_decode_plan reported), int32 lens[B] (read
 * back with pa_get_block_tables), float32 out[layers][B][Hq][D].
 * Exit status 0 on success; otherwise the failing call and pa_last_error()
 * go to stderr. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa.h"

#define CHECK_PA(call)                                                           \
  do {                                                                           \
    pa_status st_ = (call);                                                      \
    if (st_ != PA_OK) {                                                          \
      fprintf(stderr, "%s failed (%d): %s\n", #call, (int)st_, pa_last_error()); \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

#define CHECK_HIP(call)                                                                   \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                   \
      exit(1);                                                                            \
    }                                                                                     \
  } while (0)

static void read_exact(FILE* f, void* dst, size_t bytes) {
  if (bytes && fread(dst, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input\n");
    exit(1);
  }
}

static void* xmalloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL) {
    fprintf(stderr, "out of host memory\n");
    exit(1);
  }
  return p;
}

static void* to_device(const void* src, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(d, src, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[9];
  read_exact(in, hdr, sizeof hdr);
  const int32_t B = hdr[0], Hq = hdr[1], Hkv = hdr[2], D = hdr[3], BS = hdr[4], NB = hdr[5];
  const int32_t layers = hdr[6], max_seq_len = hdr[7], pt = hdr[8];
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || BS < 1 || NB < 1 || layers != 2 || max_seq_len < 1) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  int32_t* lens = xmalloc(sizeof(int32_t) * B);
  int32_t* order = xmalloc(sizeof(int32_t) * NB);
  read_exact(in, lens, sizeof(int32_t) * B);
  read_exact(in, order, sizeof(int32_t) * NB);
  int64_t rows = 0;
  int32_t max_len = 0;
  for (int32_t s = 0; s < B; ++s) {
    if (lens[s] < 1 || lens[s] > max_seq_len) {
      fprintf(stderr, "bad length\n");
      return 1;
    }
    rows += lens[s];
    if (lens[s] > max_len) max_len = lens[s];
  }
  const size_t qn = (size_t)B * Hq * D, rown = (size_t)Hkv * D;
  float* q = xmalloc(sizeof(float) * qn * layers);
  float* k = xmalloc(sizeof(float) * rown * rows * layers);
  float* v = xmalloc(sizeof(float) * rown * rows * layers);
  read_exact(in, q, sizeof(float) * qn * layers);
  read_exact(in, k, sizeof(float) * rown * rows * layers);
  read_exact(in, v, sizeof(float) * rown * rows * layers);
  fclose(in);

  /* the pool over caller-owned device memory */
  pa_pool_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.num_layers = layers;
  desc.num_blocks = NB;
  desc.block_size = BS;
  desc.num_kv_heads = Hkv;
  desc.head_dim = D;
  desc.kv_dtype = PA_F32;
  desc.layout = PA_PAGED;
  desc.max_seqs = B;
  desc.max_seq_len = max_seq_len;
  const size_t cache_bytes = pa_cache_bytes(&desc);
  if (cache_bytes == 0) {
    fprintf(stderr, "pa_cache_bytes: invalid descriptor\n");
    return 1;
  }
  void* cache = NULL;
  CHECK_HIP(hipMalloc(&cache, cache_bytes));
  pa_pool* pool = NULL;
  CHECK_PA(pa_create_pool(&desc, cache, &pool));
  CHECK_PA(pa_set_free_order(pool, order, NB));
  int32_t* rids = xmalloc(sizeof(int32_t) * B);
  for (int32_t s = 0; s < B; ++s) CHECK_PA(pa_seq_add(pool, &rids[s]));

  /* every token but the last: slots request by request, position order,
   * which is the order of the logical rows */
  int32_t* counts = xmalloc(sizeof(int32_t) * B);
  int64_t pre = 0;
  for (int32_t s = 0; s < B; ++s) {
    counts[s] = lens[s] - 1;
    pre += counts[s];
  }
  int32_t n_cow = 0;
  if (pre > 0) {
    int32_t* slots = xmalloc(sizeof(int32_t) * pre);
    CHECK_PA(pa_reserve(pool, rids, B, counts, slots, pre, NULL, 0, &n_cow));
    float* kp = xmalloc(sizeof(float) * rown * pre);
    float* vp = xmalloc(sizeof(float) * rown * pre);
    int32_t* d_slots = to_device(slots, sizeof(int32_t) * pre);
    for (int32_t l = 0; l < layers; ++l) {
      int64_t src = 0, dst = 0;
      for (int32_t s = 0; s < B; ++s) {
        const size_t n = (size_t)counts[s] * rown;
        memcpy(kp + dst * rown, k + ((size_t)l * rows + src) * rown, sizeof(float) * n);
        memcpy(vp + dst * rown, v + ((size_t)l * rows + src) * rown, sizeof(float) * n);
        src += lens[s];
        dst += counts[s];
      }
      float* dk = to_device(kp, sizeof(float) * rown * pre);
      float* dv = to_device(vp, sizeof(float) * rown * pre);
      CHECK_PA(pa_append_kv(pool, l, dk, dv, d_slots, (int32_t)pre, NULL));
      CHECK_HIP(hipDeviceSynchronize());
      CHECK_HIP(hipFree(dk));
      CHECK_HIP(hipFree(dv));
    }
    CHECK_HIP(hipFree(d_slots));
    free(slots);
    free(kp);
    free(vp);
  }

  /* the decode step: one token each, appended inside the decode launch */
  int32_t* step_slots = xmalloc(sizeof(int32_t) * B);
  int32_t* pairs = xmalloc(sizeof(int32_t) * 2 * B);
  CHECK_PA(pa_reserve(pool, rids, B, NULL, step_slots, B, pairs, B, &n_cow));
  if (n_cow != 0) {
    fprintf(stderr, "unexpected copy-on-write\n");
    return 1;
  }
  const int32_t stride = (max_len + BS - 1) / BS;
  int32_t* tables = xmalloc(sizeof(int32_t) * B * stride);
  int32_t* got_lens = xmalloc(sizeof(int32_t) * B);
  CHECK_PA(pa_get_block_tables(pool, rids, B, stride, tables, got_lens));
  CHECK_PA(pa_check_decode_args(pool, tables, stride, NULL, got_lens, step_slots, B, max_len));
  int32_t* d_tables = to_device(tables, sizeof(int32_t) * B * stride);
  int32_t* d_lens = to_device(got_lens, sizeof(int32_t) * B);
  int32_t* d_slots = to_device(step_slots, sizeof(int32_t) * B);

  const size_t ws_bytes = pa_decode_workspace_bytes(pool, B, Hq, max_len, pt);
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));
  const float scale = 1.0f / sqrtf((float)D);
  float* out = xmalloc(sizeof(float) * qn * layers);
  float* knew = xmalloc(sizeof(float) * rown * B);
  float* vnew = xmalloc(sizeof(float) * rown * B);
  int32_t planned = 0;
  for (int32_t l = 0; l < layers; ++l) {
    int64_t off = 0;
    for (int32_t s = 0; s < B; ++s) {
      off += lens[s];
      memcpy(knew + (size_t)s * rown, k + ((size_t)l * rows + off - 1) * rown, sizeof(float) * rown);
      memcpy(vnew + (size_t)s * rown, v + ((size_t)l * rows + off - 1) * rown, sizeof(float) * rown);
    }
    float* d_k = to_device(knew, sizeof(float) * rown * B);
    float* d_v = to_device(vnew, sizeof(float) * rown * B);
    float* d_q = to_device(q + (size_t)l * qn, sizeof(float) * qn);
    float* d_out = NULL;
    CHECK_HIP(hipMalloc((void**)&d_out, sizeof(float) * qn));
    if (l == 0) {
      CHECK_PA(pa_append_decode(pool, l, d_k, d_v, d_slots, d_q, PA_F32, Hq, scale, d_tables, stride, NULL,
                                d_lens, B, max_len, pt, d_out, ws, ws_bytes, NULL));
    } else {
      CHECK_PA(pa_decode_plan(pool, d_lens, B, Hq, max_len, pt, ws, ws_bytes, &planned, NULL));
      CHECK_PA(pa_append_decode_planned(pool, l, d_k, d_v, d_slots, d_q, PA_F32, Hq, scale, d_tables, stride,
                                        NULL, d_lens, B, max_len, pt, d_out, ws, ws_bytes, NULL));
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out + (size_t)l * qn, d_out, sizeof(float) * qn, hipMemcpyDeviceToHost));
    CHECK_HIP(hipFree(d_k));
    CHECK_HIP(hipFree(d_v));
    CHECK_HIP(hipFree(d_q));
    CHECK_HIP(hipFree(d_out));
  }

  FILE* o = fopen(argv[2], "wb");
  if (o == NULL || fwrite(&planned, sizeof planned, 1, o) != 1 ||
      fwrite(got_lens, sizeof(int32_t), B, o) != (size_t)B ||
      fwrite(out, sizeof(float), qn * layers, o) != qn * layers) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(o);
  CHECK_PA(pa_destroy_pool(pool));
  CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipFree(d_tables));
  CHECK_HIP(hipFree(d_lens));
  CHECK_HIP(hipFree(d_slots));
  CHECK_HIP(hipFree(cache));
  return 0;
}
