/*
 * msa.h -- C ABI of the MI355X (gfx950) MSA main-attention library, libmsa.so.
 *
 * MSA main attention (MiniMax M3): every 8-query chunk, under each index
 * head, attends only to a selected set of key blocks, with causal and
 * per-document (cu_seqlens) masks.  Sources: NeMo AutoModel API pages
 * "msa_bindings" (MSAKernels: CSR builder, flat forward, local backward),
 * "kernels" (submodules: backward preprocess, main backward, postprocess,
 * task build), "msa_schedule" (MSABackwardSchedule, the walk rule and the
 * topology constants) and "msa_backward_sm100" (module description and
 * run_backward).
 *
 * Conventions shared by every call
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device memory and never synchronises; each call only enqueues kernels
 *    on the given HIP stream (NULL = the default stream) and returns.
 *  - Pointers named "device" must be device pointers, 16-byte aligned.
 *  - Layouts are THD, token-major and contiguous:
 *      q, out, dout, dq : bf16 [T, Hq, D]      (Hq = 16 * Hkv)
 *      k, v, dk, dv     : bf16 [W, Hkv, D]      (W = T unless kv_rows says otherwise)
 *      lse              : fp32 [T, Hq]          (natural log)
 *      cu_seqlens       : int32 [num_docs + 1]  (device; cu[0] = 0, non-decreasing)
 *      sel              : int32 [Hkv, C, topk]  (device; document-local key-block
 *                         ids per (index head, chunk); -1 = empty slot)
 *    Query head h belongs to index/KV head h / 16.
 *  - Selections are sets: ids outside the document, ids of blocks that start
 *    after the chunk's last query, and repeated ids add no keys, so the
 *    schedule build drops them and counts them in the schedule's error words.
 *  - Return value: an msa_status.  Host-side checks happen before anything is
 *    enqueued; MSA_ERR_HIP reports a failed launch.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID = 1,      /* NULL pointer or negative size */
  MSA_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or a size the kernels are not built for */
  MSA_ERR_SHAPE = 3,        /* sizes inconsistent with each other */
  MSA_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned */
  MSA_ERR_HIP = 5,          /* a HIP runtime call or launch failed */
  MSA_ERR_SCRATCH_LIMIT = 6 /* msa_backward_noalloc: the problem needs more scratch than
                               MSA_NOALLOC_SCRATCH_BYTES */
} msa_status;

/* Problem geometry; all fields are host integers.  num_chunks, num_kblocks
 * and max_doc_chunks must agree with cu_seqlens (the schedule build checks
 * this on the device and sets MSA_SCHED_ERR_GEOMETRY if they do not; every
 * later call on that schedule then writes NaN to all of its outputs --
 * out, lse, dq, dk, dv -- instead of computing them, so the failure shows
 * without a host synchronisation; the index scorer writes empty rows). */
typedef struct msa_problem {
  int32_t total_tokens;    /* T = cu_seqlens[num_docs] */
  int32_t num_docs;        /* >= 1 */
  int32_t num_kv_heads;    /* Hkv: index heads == KV heads (one index head per KV head) */
  int32_t q_per_kv;        /* query heads per KV head; must be 16 (8 queries x 16 heads = 128-row tile) */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t block_size;      /* B: key block size, 64 or 128 (at 128: topk <= 32; every
                              dq_mode, each block taken as two 64-key tiles) */
  int32_t query_chunk;     /* must be 8 (msa_schedule: QUERY_CHUNK) */
  int32_t topk;            /* slots per (index head, chunk); 1..64 */
  int32_t num_chunks;      /* C = sum_d ceil(len_d / 8) */
  int32_t num_kblocks;     /* R = sum_d ceil(len_d / B) */
  int32_t max_doc_chunks;  /* max_d ceil(len_d / 8); <= MSA_MAX_DOC_CHUNKS */
  int32_t num_cus;         /* compute units the walk is sized for (msa_device_check) */
  float softmax_scale;     /* usually head_dim ** -0.5 (msa_schedule: SOFTMAX_SCALE) */
  int32_t dq_mode;         /* MSA_DQ_DS_BUFFER, MSA_DQ_RECOMPUTE, MSA_DQ_ATOMIC_POOL or
                              MSA_DQ_ATOMIC_POOL_BF16 */
  int32_t kv_rows;         /* rows W of k, v, dk, dv: 0 means total_tokens (compact THD: a
                              document's keys sit at its cu_seqlens rows); with per-document K/V
                              starts (msa_build_schedule_kv) any W >= total_tokens */
} msa_problem;

/* How the backward forms dQ.
 * MSA_DQ_ATOMIC_POOL: the main kernel scatters each tile's dQ with fp32
 *   atomics into a [T, Hq, D] pool that the postprocess casts to bf16
 *   (msa_backward_sm100 page: dQ^T per tile into an atomic pool).  On MI355X
 *   fp32 global atomics execute beyond the L2 at about 0.32 G lane-ops per
 *   microsecond, so this mode is bound by the atomic rate (about 1 G
 *   lane-atomics per call on an 8K-token, 4x16-head, top-16 problem).
 * MSA_DQ_RECOMPUTE: the main kernel computes dK/dV only; msa_backward_dq runs
 *   a query-parallel kernel that recomputes S^T and dP^T per (chunk, block),
 *   accumulates dQ in registers and writes bf16 dq once (no atomics).
 * MSA_DQ_DS_BUFFER: the main kernel also stores each tile's bf16 dS (the
 *   same values the recompute mode forms) in a scratch buffer with one
 *   128 x 64 slot per (index head, chunk, selection slot); msa_backward_dq
 *   then sums dQ = scale * sum_b dS_b K_b per chunk in registers (one
 *   contraction per tile instead of three) and writes bf16 dq once. */
#define MSA_DQ_RECOMPUTE 0
#define MSA_DQ_ATOMIC_POOL 1
#define MSA_DQ_DS_BUFFER 2
/* MSA_DQ_ATOMIC_POOL_BF16: the pages' pool dtype (msa_schedule page:
 *   DQ_ACCUM_DTYPE bf16; msa_backward_sm100 page: head-pair-interleaved bf16x2
 *   atomics).  The pool is bf16 [T, Hq/2, D, 2]: element (t, h, d) at
 *   ((t * Hq/2 + h/2) * D + d) * 2 + h%2, so one packed atomic adds the dQ of
 *   two heads; each tile's scale * dQ is rounded to bf16 and summed in bf16
 *   (less accurate than the fp32 pool; half its atomic operations). */
#define MSA_DQ_ATOMIC_POOL_BF16 3

#define MSA_MAX_DOC_CHUNKS (1 << 18) /* documents up to 2 Mi tokens (32 KiB LDS bitmap per bucket sort) */

/* Layout of the int32 schedule workspace (offsets in int32 elements).
 * msa_schedule: MSABackwardSchedule carries row_ptr, q_indices,
 * scheduler_metadata, work_count and cu_seqlens; this workspace holds the
 * same tables plus the cleaned selection the forward reads.
 *   desc[8]     : work_count N, rows_per_cta, num_full_walks, tail_rows,
 *                 tail_walks, grid_walks, capacity (Hkv*C*topk), 0
 *   err[8]      : [0] dropped selection slots, [1] geometry mismatch flag
 *   doc_chunk_off[num_docs+1], doc_blk_off[num_docs+1] : per-document offsets
 *   doc_kv_off[num_docs]  : first row of each document in k, v, dk, dv
 *   chunk_doc[C]          : document of each global chunk
 *   sel_clean[Hkv*C*topk] : kept ids in their slots, -1 elsewhere
 *   row_cursor[8*Hkv*R]   : build scratch (8 striped copies of the row counters)
 *   row_ptr[Hkv*(R+1)]    : k2q CSR offsets, one CSR per index head
 *   head_off[Hkv+1]       : first task row of each index head
 *   q_idx[Hkv*C*topk]     : CSR entries = document-local first query (8*c) of
 *                           each selecting chunk, ascending per row; -1 padding
 *   task_meta[Hkv*C*topk*6] : one task (128-row tile) per CSR entry, heads in
 *                           order: (index_head, row_linear, q_begin, q_count,
 *                           document_ordinal, document_local_kblock); -1 padding */
typedef struct msa_schedule_layout {
  int64_t desc, err, doc_chunk_off, doc_blk_off, doc_kv_off, chunk_doc, sel_clean, row_cursor,
      row_ptr, head_off, q_idx, task_meta, total;
} msa_schedule_layout;

#define MSA_SCHED_ERR_DROPPED 0
#define MSA_SCHED_ERR_GEOMETRY 1

/* Device gate (kernels page: require_sm100 / sm_count analog).  Returns
 * MSA_OK and the compute-unit count when `device` is a gfx950 GPU,
 * MSA_ERR_UNSUPPORTED otherwise.  Results are memoised per device. */
int msa_device_check(int device, int32_t* num_cus);

/* Offsets of every table in the schedule workspace, and its total size. */
int msa_schedule_layout_of(const msa_problem* p, msa_schedule_layout* out);

/* k2q CSR build + task build (msa_bindings: build_k2q_csr; kernels page:
 * msa_task_build; msa_schedule: MSABackwardSchedule, rows_per_cta, chunk_map).
 * Cleans the selection, inverts it into key-block buckets (row r =
 * doc_blk_off[d] + b), sorts each bucket by chunk, and writes the task table
 * and the walk descriptor.  Inputs: cu_seqlens, sel (device).  Output: sched
 * (device, msa_schedule_layout_of(...).total int32 elements). */
int msa_build_schedule(const msa_problem* p, const int32_t* cu_seqlens, const int32_t* sel,
                       int32_t* sched, void* stream);

/* msa_build_schedule for K/V held in a workspace with a start row per
 * document (msa_schedule page: MSABackwardSchedule.document_workspace_starts,
 * the 128-aligned workspace row of each document; msa_backward_sm100 page:
 * run_backward takes k_aligned, v_aligned [W, 4, 128] and returns dk, dv in
 * the same rows, zero outside the documents).  kv_starts (device int32
 * [num_docs]) gives the row of k / v that holds each document's first key;
 * documents must lie in order without overlap inside the problem's kv_rows
 * rows (kv_starts[d] + len_d <= kv_starts[d+1], last one <= kv_rows), else
 * the schedule's MSA_SCHED_ERR_GEOMETRY word is set and the later calls
 * write NaN to their outputs.  Every later call then reads k, v and
 * writes dk, dv ([kv_rows, Hkv, D]) at those rows; dk and dv rows that hold
 * no attended key, including every row between documents, are exactly 0.
 * kv_starts = NULL gives the compact layout (kv_starts[d] = cu_seqlens[d]),
 * which is what msa_build_schedule does.  Starts need not be multiples of
 * 128; the pages' aligned workspace is one valid placement. */
int msa_build_schedule_kv(const msa_problem* p, const int32_t* cu_seqlens, const int32_t* sel,
                          const int32_t* kv_starts, int32_t* sched, void* stream);

/* Sparse forward (msa_bindings: the flat forward sparse_atten_func; its
 * outputs are the out/lse that run_backward consumes).  For every
 * (chunk, index head): online softmax over the chunk's kept key blocks with
 * the causal mask; writes out (bf16) and lse (fp32, natural log; -inf and
 * out = 0 where a query sees no key).  `sched` must come from
 * msa_build_schedule on the same cu_seqlens and selection. */
int msa_forward(const msa_problem* p, const void* q, const void* k, const void* v,
                const int32_t* cu_seqlens, const int32_t* sched, void* out, float* lse,
                void* stream);

/* Planner-driven (KV-parallel) forward: the same out and lse as msa_forward,
 * computed by walking the schedule's task table (one work item per k2q CSR
 * entry, msa_schedule page: scheduler_metadata; msa_bindings page: the
 * planner fmha_sm100_plan beside the flat forward) the way the backward does,
 * key block resident per bucket.  A chunk's blocks then sit in different
 * workgroups, so the softmax is reduced across them exactly: a statistics
 * pass (per slot and query row, the block's max and exp-sum), a merge into
 * the LSE, an output pass with the final probabilities whose O is added into
 * an fp32 pool with atomics, and a cast.  Slower than msa_forward on MI355X
 * (two passes over S, one fp32 atomic per output element per block); key
 * block 64 only (MSA_ERR_UNSUPPORTED otherwise).
 *   scratch : msa_forward_kv_scratch_bytes bytes (device, 16-byte aligned):
 *             float2 [Hkv, C, topk, 128] statistics and the fp32 pool
 *             [T, Hq, D] (8K tokens x 64 heads x 128: 256 MiB + 64 MiB). */
int msa_forward_kv_scratch_bytes(const msa_problem* p, size_t* bytes);
int msa_forward_kv(const msa_problem* p, const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens, const int32_t* sched, void* scratch, void* out,
                   float* lse, void* stream);

/* Bytes of scratch msa_backward needs: fp32 Delta [T, Hq], fp32 dK and dV
 * accumulators [kv_rows, Hkv, D]; in MSA_DQ_ATOMIC_POOL mode the fp32 dQ pool
 * [T, Hq, D]; in MSA_DQ_DS_BUFFER mode the bf16 dS slots
 * [Hkv, C, topk, block_size / 64, 128, 64] (16 KiB per selection slot and
 * 64-key tile); in MSA_DQ_ATOMIC_POOL_BF16 mode the bf16 pool [T, Hq/2, D, 2].
 * With 4 x 16 heads and head dim 128, MSA_DQ_DS_BUFFER needs about 1 GiB for
 * an 8K-token top-16 problem, 16 GiB for a 64K-token top-32 problem and twice
 * that at key block 128; MSA_DQ_RECOMPUTE needs 34 MiB and 272 MiB. */
int msa_backward_scratch_bytes(const msa_problem* p, size_t* bytes);

/* KV-parallel backward (msa_backward_sm100: run_backward): preprocess
 * (Delta = rowsum(dout * out), zero the accumulators), main kernel (per walk
 * of task rows: K/V resident per bucket, bf16 MFMA contractions S^T, dP^T,
 * dV, dK per 128-row tile, dK/dV flushed per bucket segment with fp32
 * atomics; in MSA_DQ_ATOMIC_POOL mode also dQ^T per tile scattered into the
 * pool; in MSA_DQ_DS_BUFFER mode also each tile's bf16 dS into its slot),
 * the dQ kernel (MSA_DQ_RECOMPUTE and MSA_DQ_DS_BUFFER modes), postprocess
 * (cast to bf16).
 * dk/dv rows that no query attends are exactly 0. */
int msa_backward(const msa_problem* p, const void* q, const void* k, const void* v,
                 const void* out, const void* dout, const float* lse, const int32_t* cu_seqlens,
                 const int32_t* sched, void* scratch, void* dq, void* dk, void* dv, void* stream);

/* msa_backward without the scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The scratch is a static device array of
 * MSA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends; this call allocates nothing.  Arguments, layouts and the
 * result are those of msa_backward.  Returns MSA_ERR_SCRATCH_LIMIT, before
 * anything is enqueued, when msa_backward_scratch_bytes(p) exceeds the
 * array (64 MiB: with dq_mode MSA_DQ_RECOMPUTE an 8K-token, 4 x 16-head,
 * head-dim-128 problem needs 34 MiB; the MSA_DQ_DS_BUFFER slots alone need
 * 16 KiB per selection slot, so that mode fits small problems only).  All
 * calls on one GPU share its array: calls that overlap on one GPU race. */
#define MSA_NOALLOC_SCRATCH_BYTES (64u << 20)
int msa_backward_noalloc(const msa_problem* p, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse,
                         const int32_t* cu_seqlens, const int32_t* sched, void* dq, void* dk,
                         void* dv, void* stream);

/* The steps of msa_backward, callable one at a time (same arguments and
 * scratch; used to time each kernel).  Order: preprocess, main, dq,
 * postprocess.  msa_backward_dq writes dq directly and does nothing in the
 * two pool modes; msa_backward_postprocess writes dq only in those modes. */
int msa_backward_preprocess(const msa_problem* p, const void* out, const void* dout,
                            void* scratch, void* stream);
int msa_backward_main(const msa_problem* p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, const int32_t* cu_seqlens,
                      const int32_t* sched, void* scratch, void* stream);
int msa_backward_dq(const msa_problem* p, const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, const int32_t* cu_seqlens,
                    const int32_t* sched, const void* scratch, void* dq, void* stream);
int msa_backward_postprocess(const msa_problem* p, const int32_t* sched, const void* scratch,
                             void* dq, void* dk, void* dv, void* stream);

/* Index scorer and top-k block selection: the step that produces `sel`.
 * msa_bindings: MSAKernels lists the scorer (fmha_sm100) beside the planner;
 * msa_schedule, module data: INDEX_DIM 128, NUM_INDEX_HEADS 4 (one index
 * head per KV head here), TOPK_BLOCKS.  The pages do not define the scoring
 * function; this library's reading, per index head i and chunk c:
 *   score(c, b) = (sum of the chunk's index queries) . (mean of the index
 *                 keys of key block b), over the tokens of c's document;
 *   sel[i, c] = {diagonal block of c} + the topk - 1 best-scoring earlier
 *               blocks (ties to the smaller id; fewer when fewer exist),
 *               ascending, -1 padding.
 * Sums and the dot product are fp32 (a score differs from the exact one by
 * a few 1e-6 of sum_x |qsum_x| mean|k_x|, so near-ties may order either way).
 *   qi, ki  : bf16 [T, Hkv, MSA_INDEX_DIM] index queries / keys (device)
 *   scratch : msa_index_scratch_bytes bytes (device, 16-byte aligned)
 *   sel     : int32 [Hkv, C, topk] (device), written in full
 * Documents may hold at most MSA_INDEX_MAX_DOC_BLOCKS key blocks
 * (MSA_ERR_UNSUPPORTED otherwise).  cu_seqlens that disagree with the host
 * sizes leave every row empty (-1). */
#define MSA_INDEX_DIM 128
#define MSA_INDEX_MAX_DOC_BLOCKS 4096
int msa_index_scratch_bytes(const msa_problem* p, size_t* bytes);
int msa_index_select(const msa_problem* p, const void* qi, const void* ki, const int32_t* cu_seqlens,
                     void* scratch, int32_t* sel, void* stream);

/* Number of walks the main backward kernels are sized for (msa_schedule:
 * grid_launch_bound(capacity, num_cus), capacity = Hkv * C * topk); they
 * launch one workgroup per walk, or one per walk and query half (KV-parallel
 * kernel) or per walk and 64-key half (atomic-pool kernel at key block 128);
 * workgroups past desc's grid_walks return at once. */
int64_t msa_grid_launch_bound(int64_t capacity, int32_t num_cus);

const char* msa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
