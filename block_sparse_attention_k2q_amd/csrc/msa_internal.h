// Host-side internals of libmsa: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Walk rule constants (msa_schedule page: ROWS_PER_CTA_SMALL / _LARGE / _SWITCH).
constexpr int kRowsPerWalkSmall = 4;
constexpr int kRowsPerWalkLarge = 64;
constexpr int kRowsPerWalkSwitch = 2400;

// The schedule build counts and places CSR entries with integer atomics;
// popular rows (early key blocks) take hundreds of them, which serialise
// per address, so every row has this many counter copies (chosen by the
// workgroup id) and the scan adds them up.
constexpr int kCounterCopies = 8;

// One dS slot of the MSA_DQ_DS_BUFFER mode: 128 tile rows x 64 keys, bf16
// (a selected block of 128 keys takes two).
constexpr int kDsSlotBytes = 128 * 64 * 2;

inline int64_t align64(int64_t x) { return (x + 63) & ~int64_t(63); }

// Offsets (int32 elements) of the schedule workspace tables; see msa.h.
inline msa_schedule_layout schedule_layout(const msa_problem& p) {
  const int64_t hkv = p.num_kv_heads, C = p.num_chunks, K = p.topk, R = p.num_kblocks;
  const int64_t cap = hkv * C * K;
  msa_schedule_layout L;
  int64_t o = 0;
  L.desc = o; o += 8;
  L.err = o; o += 8;
  o = align64(o);
  L.doc_chunk_off = o; o = align64(o + p.num_docs + 1);
  L.doc_blk_off = o; o = align64(o + p.num_docs + 1);
  L.doc_kv_off = o; o = align64(o + p.num_docs);
  L.chunk_doc = o; o = align64(o + C);
  L.sel_clean = o; o = align64(o + cap);
  L.row_cursor = o; o = align64(o + kCounterCopies * hkv * R);
  L.row_ptr = o; o = align64(o + hkv * (R + 1));
  L.head_off = o; o = align64(o + hkv + 1);
  L.q_idx = o; o = align64(o + cap);
  L.task_meta = o; o = align64(o + cap * 6);
  L.total = o;
  return L;
}

inline int64_t grid_launch_bound(int64_t cap, int num_cus) {
  const int64_t small = (cap < kRowsPerWalkSwitch - 1 ? cap : kRowsPerWalkSwitch - 1) / kRowsPerWalkSmall;
  const int64_t large = cap >= kRowsPerWalkSwitch ? cap / kRowsPerWalkLarge : 0;
  return (small > large ? small : large) + num_cus;
}

// Scratch layout of the backward (bytes, 256-aligned): Delta, dK, dV
// accumulators (adjacent, so one range clears both), and the dQ pool in
// MSA_DQ_ATOMIC_POOL mode (dq_pool == total otherwise).
struct BackwardScratch {
  size_t delta, dk_acc, dv_acc, dq_pool, ds, total;
};
// Rows of k, v, dk, dv (msa.h: kv_rows, 0 = compact).
inline int64_t kv_rows_of(const msa_problem& p) { return p.kv_rows > 0 ? p.kv_rows : p.total_tokens; }

inline BackwardScratch backward_scratch_layout(const msa_problem& p) {
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t T = (size_t)p.total_tokens, hq = (size_t)p.num_kv_heads * p.q_per_kv,
               hkv = (size_t)p.num_kv_heads, D = (size_t)p.head_dim, W = (size_t)kv_rows_of(p);
  BackwardScratch s;
  size_t o = 0;
  s.delta = o; o = a256(o + 4 * T * hq);
  s.dk_acc = o; o = a256(o + 4 * W * hkv * D);
  s.dv_acc = o; o = a256(o + 4 * W * hkv * D);
  s.dq_pool = o;
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL) o = a256(o + 4 * T * hq * D);
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL_BF16) o = a256(o + 2 * T * hq * D);
  s.ds = o;
  if (p.dq_mode == MSA_DQ_DS_BUFFER)
    o = a256(o + (size_t)kDsSlotBytes * hkv * (size_t)p.num_chunks * (size_t)p.topk * (size_t)(p.block_size / 64));
  s.total = o;
  return s;
}

// Scratch of the planner-driven forward (bytes, 256-aligned): per selection
// slot and query row (m, l) as float2 [Hkv, C, topk, 128], and the fp32
// output pool [T, Hq, D].
struct ForwardKvScratch {
  size_t stats, pool, total;
};
inline ForwardKvScratch forward_kv_scratch_layout(const msa_problem& p) {
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  ForwardKvScratch s;
  size_t o = 0;
  s.stats = o; o = a256(o + 8 * (size_t)p.num_kv_heads * p.num_chunks * p.topk * 128);
  s.pool = o; o = a256(o + 4 * (size_t)p.total_tokens * p.num_kv_heads * p.q_per_kv * p.head_dim);
  s.total = o;
  return s;
}

// Index scorer (scorer.hip): index dimension and the most earlier blocks a
// chunk can choose from (one LDS score per candidate per wave).
constexpr int kIndexDim = MSA_INDEX_DIM;
constexpr int kMaxIndexCandidates = MSA_INDEX_MAX_DOC_BLOCKS;

// Scratch of the index scorer (bytes, 256-aligned): per-document offsets and
// an error word (int32), chunk query sums fp32 [H, C, kIndexDim], block key
// means fp32 [H, R, kIndexDim].
struct IndexScratch {
  size_t geo, qsum, kbar, total;
};
inline IndexScratch index_scratch_layout(const msa_problem& p) {
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  IndexScratch s;
  size_t o = 0;
  s.geo = o; o = a256(o + 4 * (2 * (size_t)p.num_docs + 2 + 8));
  s.qsum = o; o = a256(o + 4 * (size_t)p.num_kv_heads * p.num_chunks * kIndexDim);
  s.kbar = o; o = a256(o + 4 * (size_t)p.num_kv_heads * p.num_kblocks * kIndexDim);
  s.total = o;
  return s;
}

hipError_t launch_index_select(const msa_problem& p, const void* qi, const void* ki, const int32_t* cu,
                               void* scratch, int32_t* sel, hipStream_t stream);

hipError_t launch_build_schedule(const msa_problem& p, const int32_t* cu, const int32_t* sel,
                                 const int32_t* kv_starts, int32_t* sched, const msa_schedule_layout& L,
                                 hipStream_t stream);
hipError_t launch_forward(const msa_problem& p, const void* q, const void* k, const void* v,
                          const int32_t* cu, const int32_t* sched, const msa_schedule_layout& L,
                          void* out, float* lse, hipStream_t stream);
hipError_t launch_forward_kv(const msa_problem& p, const void* q, const void* k, const void* v,
                             const int32_t* cu, const int32_t* sched, const msa_schedule_layout& L,
                             void* scratch, void* out, float* lse, hipStream_t stream);
hipError_t launch_backward_preprocess(const msa_problem& p, const void* out, const void* dout,
                                      void* scratch, hipStream_t stream);
hipError_t launch_backward_main(const msa_problem& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const int32_t* cu,
                                const int32_t* sched, const msa_schedule_layout& L, void* scratch,
                                hipStream_t stream);
hipError_t launch_backward_dq(const msa_problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const int32_t* cu,
                              const int32_t* sched, const msa_schedule_layout& L, const void* scratch,
                              void* dq, hipStream_t stream);
hipError_t launch_dq_recompute(const msa_problem& p, const void* q, const void* k, const void* v,
                               const void* dout, const float* lse, const int32_t* cu, const int32_t* sched,
                               const msa_schedule_layout& L, const void* scratch, void* dq,
                               hipStream_t stream);
hipError_t launch_backward_postprocess(const msa_problem& p, const int32_t* sched,
                                       const msa_schedule_layout& L, const void* scratch, void* dq, void* dk,
                                       void* dv, hipStream_t stream);

}  // namespace msa
