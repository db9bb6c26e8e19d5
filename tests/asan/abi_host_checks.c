/* Host-side checks of the libmsa C ABI, built with AddressSanitizer on the
 * host code (no GPU needed): every entry point rejects null, misaligned and
 * inconsistent arguments before it touches the device, the layout and
 * scratch queries agree with each other, and the allocation-free backward
 * refuses problems beyond its static scratch.  Exit status 0 when every
 * expectation holds; the sanitizer aborts the run on any bad access. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "msa.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static msa_problem problem_8k(void) {
  msa_problem p;
  memset(&p, 0, sizeof p);
  p.total_tokens = 8192;
  p.num_docs = 1;
  p.num_kv_heads = 4;
  p.q_per_kv = 16;
  p.head_dim = 128;
  p.block_size = 64;
  p.query_chunk = 8;
  p.topk = 16;
  p.num_chunks = 1024;
  p.num_kblocks = 128;
  p.max_doc_chunks = 1024;
  p.num_cus = 256;
  p.softmax_scale = 0.0883883f;
  p.dq_mode = MSA_DQ_DS_BUFFER;
  p.kv_rows = 0;
  return p;
}

int main(void) {
  msa_problem p = problem_8k();
  msa_schedule_layout L;
  size_t bytes = 0, bytes2 = 0;
  int st;

  for (int s = 0; s <= 7; ++s) EXPECT(msa_status_string(s) != NULL && msa_status_string(s)[0] != 0);

  /* layout: consistent, increasing, sized for the task table */
  EXPECT(msa_schedule_layout_of(&p, &L) == MSA_OK);
  EXPECT(L.desc == 0 && L.err > L.desc && L.doc_chunk_off > L.err && L.doc_blk_off > L.doc_chunk_off);
  EXPECT(L.doc_kv_off > L.doc_blk_off && L.chunk_doc > L.doc_kv_off && L.sel_clean > L.chunk_doc);
  EXPECT(L.row_cursor > L.sel_clean && L.row_ptr > L.row_cursor && L.head_off > L.row_ptr);
  EXPECT(L.q_idx > L.head_off && L.task_meta > L.q_idx);
  EXPECT(L.total >= L.task_meta + (int64_t)4 * 1024 * 16 * 6);
  EXPECT(msa_schedule_layout_of(NULL, &L) == MSA_ERR_INVALID);
  EXPECT(msa_schedule_layout_of(&p, NULL) == MSA_ERR_INVALID);

  /* inconsistent or unsupported problems */
  msa_problem b = p; b.head_dim = 96;   EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_UNSUPPORTED);
  b = p; b.q_per_kv = 8;                EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_UNSUPPORTED);
  b = p; b.topk = 65;                   EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_UNSUPPORTED);
  b = p; b.block_size = 128; b.num_kblocks = 64; b.dq_mode = MSA_DQ_RECOMPUTE;
  EXPECT(msa_schedule_layout_of(&b, &L) == MSA_OK);   /* key block 128: every dQ mode */
  b.topk = 33;                          EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_UNSUPPORTED);
  b = p; b.num_kblocks = 63;            EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_SHAPE);
  b = p; b.kv_rows = 8191;              EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_SHAPE);
  b = p; b.kv_rows = -1;                EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_INVALID);
  b = p; b.num_docs = 0;                EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_INVALID);
  b = p; b.softmax_scale = 0.f;         EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_INVALID);
  b = p; b.dq_mode = 9;                 EXPECT(msa_schedule_layout_of(&b, &L) == MSA_ERR_INVALID);

  /* scratch sizes: recompute mode has no dS slots; a wider K/V workspace
   * grows the fp32 dK / dV accumulators */
  EXPECT(msa_backward_scratch_bytes(&p, &bytes) == MSA_OK);
  b = p; b.dq_mode = MSA_DQ_RECOMPUTE;
  EXPECT(msa_backward_scratch_bytes(&b, &bytes2) == MSA_OK);
  EXPECT(bytes == bytes2 + (size_t)16384 * 4 * 1024 * 16);
  EXPECT(bytes2 <= MSA_NOALLOC_SCRATCH_BYTES);
  b.kv_rows = 16384;
  EXPECT(msa_backward_scratch_bytes(&b, &bytes) == MSA_OK && bytes == bytes2 + (size_t)2 * 4 * 8192 * 4 * 128);
  EXPECT(msa_backward_scratch_bytes(&p, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_forward_kv_scratch_bytes(&p, &bytes) == MSA_OK && bytes >= (size_t)4 * 8192 * 64 * 128);
  b = p; b.block_size = 128; b.num_kblocks = 64;
  EXPECT(msa_forward_kv_scratch_bytes(&b, &bytes) == MSA_ERR_UNSUPPORTED);
  EXPECT(msa_index_scratch_bytes(&p, &bytes) == MSA_OK && bytes > 0);
  EXPECT(msa_grid_launch_bound(65536, 256) == 65536 / 64 + 256);
  EXPECT(msa_grid_launch_bound(100, 256) == 25 + 256);
  EXPECT(msa_grid_launch_bound(-1, 256) == -1 && msa_grid_launch_bound(10, 0) == -1);

  /* every launching entry point rejects null and misaligned pointers before
   * it touches the device */
  char buf[64] __attribute__((aligned(16)));
  void* ok = buf;
  void* mis = buf + 4;
  int32_t* oki = (int32_t*)buf;
  int32_t* misi = (int32_t*)(buf + 4);
  EXPECT(msa_build_schedule(&p, NULL, oki, oki, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_build_schedule(&p, oki, oki, misi, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_build_schedule_kv(&p, oki, oki, NULL, misi, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_forward(&p, NULL, ok, ok, oki, oki, ok, (float*)ok, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_forward(&p, mis, ok, ok, oki, oki, ok, (float*)ok, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_forward_kv(&p, ok, ok, ok, oki, oki, NULL, ok, (float*)ok, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_forward_kv(&p, ok, ok, ok, oki, oki, mis, ok, (float*)ok, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_backward(&p, ok, ok, ok, ok, ok, (float*)ok, oki, oki, NULL, ok, ok, ok, NULL) ==
         MSA_ERR_INVALID);
  EXPECT(msa_backward_preprocess(&p, ok, mis, ok, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_backward_main(&p, ok, ok, ok, ok, (float*)mis, oki, oki, ok, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_backward_dq(&p, ok, ok, ok, ok, (float*)ok, oki, oki, ok, NULL, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_backward_postprocess(&p, NULL, ok, ok, ok, ok, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_index_select(&p, mis, ok, oki, ok, oki, NULL) == MSA_ERR_ALIGN);
  EXPECT(msa_backward_noalloc(&p, ok, ok, ok, ok, ok, (float*)ok, oki, oki, ok, ok, ok, NULL) ==
         MSA_ERR_SCRATCH_LIMIT);   /* the dS slots of this problem need 1 GiB */
  EXPECT(msa_device_check(-1, NULL) == MSA_ERR_INVALID);
  EXPECT(msa_device_check(64, NULL) == MSA_ERR_INVALID);

  st = failures ? 1 : 0;
  printf("abi host checks: %d failure(s)\n", failures);
  return st;
}
