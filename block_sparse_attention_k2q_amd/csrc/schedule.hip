// k2q CSR builder and task builder (gfx950).
//
// Pages: msa_bindings (build_k2q_csr, the CSR builder), msa_schedule
// (MSABackwardSchedule: row_ptr [heads, rows+1], q_indices = document-local
// query positions, scheduler_metadata columns (index_head, row_linear,
// q_begin, q_count, document_ordinal, document_local_kblock), work_count;
// rows_per_cta / chunk_map / grid_launch_bound and ROWS_PER_CTA_*), kernels
// page (msa_task_build mirrors the walk rule on the device).
//
// Pipeline, all on one stream, no host synchronisation:
//   geometry   workgroup 0: per-document chunk/block offsets and K/V start
//              rows, checks them against the host sizes, clears the error
//              words; the other workgroups clear the row counters.
//   clean      one thread per (head, chunk, slot): keeps an id when it names
//              a block of the document that starts at or before the chunk's
//              last query and no earlier slot holds it; counts kept ids per
//              key-block row with integer atomics (order-free, exact) into
//              one of kCounterCopies copies picked by the workgroup id.
//   scan       one workgroup: sums the copies, exclusive scan of the row
//              counts -> row_ptr, per-head task offsets, the walk
//              descriptor, and each copy's fill cursor inside its row.
//   fill       one thread per (head, chunk, slot), same workgroups as clean:
//              places each kept entry in its row through its copy's atomic
//              cursor (order inside a row is not yet fixed) and writes the -1
//              padding.
//   sort       one workgroup per (head, row): a bitmap over the document's
//              chunks orders the row's entries ascending (entries of a row
//              are distinct chunks), then writes the ordered q_idx and one
//              task per entry.  The result is independent of atomic order.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int block_inclusive_scan(int x, int* s_warp, int* total) {
  return block_inclusive_scan_n<kThreads>(x, s_warp, total);
}

constexpr int kZeroPerBlock = 16 * kThreads;   // counters cleared per extra workgroup

__global__ __launch_bounds__(kThreads) void geometry_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ kv_starts, int num_docs, int T, int W, int C,
    int R, int B, int max_doc_chunks, int32_t* __restrict__ doc_chunk_off, int32_t* __restrict__ doc_blk_off,
    int32_t* __restrict__ doc_kv_off, int32_t* __restrict__ desc, int32_t* __restrict__ err,
    int32_t* __restrict__ row_cursor, int64_t n_cursor) {
  __shared__ int s_warp[kThreads / 64];
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const int64_t x0 = (int64_t)(blockIdx.x - 1) * kZeroPerBlock;
    for (int x = tid; x < kZeroPerBlock; x += kThreads)
      if (x0 + x < n_cursor) row_cursor[x0 + x] = 0;
    return;
  }
  if (tid < 8) { desc[tid] = 0; err[tid] = 0; }
  int bad = 0;
  int carry_c = 0, carry_b = 0;
  for (int base = 0; base < num_docs; base += kThreads) {
    const int d = base + tid;
    int nc = 0, nb = 0;
    if (d < num_docs) {
      const int a = cu[d], e = cu[d + 1];
      int len = e - a;
      if (len < 0 || a < 0) bad = 1;
      len = len < 0 ? 0 : len;
      nc = (len + kChunk - 1) / kChunk;
      nb = (len + B - 1) / B;
      if (nc > max_doc_chunks) bad = 1;
      // K/V rows of the document: its own cu_seqlens rows, or its start in a
      // workspace, in document order without overlap, inside the W rows
      const int kv0 = kv_starts ? kv_starts[d] : a;
      const int kv_end = d + 1 < num_docs ? (kv_starts ? kv_starts[d + 1] : e) : W;
      if (kv0 < 0 || (int64_t)kv0 + len > kv_end) bad = 1;
      doc_kv_off[d] = kv0;
    }
    int tc, tb;
    const int ic = block_inclusive_scan(nc, s_warp, &tc);
    const int ib = block_inclusive_scan(nb, s_warp, &tb);
    if (d < num_docs) {
      doc_chunk_off[d] = carry_c + ic - nc;
      doc_blk_off[d] = carry_b + ib - nb;
    }
    carry_c += tc;
    carry_b += tb;
  }
  if (tid == 0) {
    doc_chunk_off[num_docs] = carry_c;
    doc_blk_off[num_docs] = carry_b;
    if (carry_c != C || carry_b != R || cu[0] != 0 || cu[num_docs] != T) bad = 1;
  }
  bad = __syncthreads_or(bad);
  if (tid == 0 && bad) err[1] = 1;
}

__global__ __launch_bounds__(kThreads) void clean_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ sel, int Hkv, int C, int K, int R, int B,
    int num_docs, const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ doc_blk_off,
    int32_t* __restrict__ chunk_doc, int32_t* __restrict__ sel_clean, int32_t* __restrict__ row_count,
    int32_t* __restrict__ err) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)Hkv * C * K;
  int32_t* counts = row_count + (int64_t)(blockIdx.x % kCounterCopies) * Hkv * R;
  bool dropped_slot = false;
  if (idx < total) {
    const int s = (int)(idx % K);
    const int g = (int)((idx / K) % C);
    const int i = (int)(idx / ((int64_t)K * C));
    const bool geom_ok = err[1] == 0;
    int d = upper_bound_minus1(doc_chunk_off, num_docs + 1, g);
    d = d < num_docs ? d : num_docs - 1;
    const int c = g - doc_chunk_off[d];
    const int len = cu[d + 1] - cu[d];
    const int nb = (len + B - 1) / B;
    const int last_q = min(kChunk * c + kChunk - 1, len - 1);
    const int b = sel[idx];
    bool keep = geom_ok && b >= 0 && b < nb && b * B <= last_q && doc_blk_off[d] + b < R;
    if (keep) {
      const int32_t* row = sel + (idx - s);
      for (int s2 = 0; s2 < s; ++s2)
        if (row[s2] == b) { keep = false; break; }
    }
    sel_clean[idx] = keep ? b : -1;
    if (i == 0 && s == 0) chunk_doc[g] = d;
    if (keep) atomicAdd(&counts[(int64_t)i * R + doc_blk_off[d] + b], 1);
    dropped_slot = b != -1 && !keep;
  }
  // dropped slots: one atomic per workgroup (every thread reaches this barrier)
  const int dropped = __syncthreads_count(dropped_slot);
  if (threadIdx.x == 0 && dropped) atomicAdd(&err[0], dropped);
}

__global__ __launch_bounds__(kThreads) void scan_kernel(
    int Hkv, int R, int64_t cap, int num_cus, int32_t* __restrict__ row_cursor,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ head_off, int32_t* __restrict__ desc) {
  __shared__ int s_warp[kThreads / 64];
  const int tid = threadIdx.x;
  int n_total = 0;
  const int64_t HR = (int64_t)Hkv * R;
  for (int i = 0; i < Hkv; ++i) {
    int32_t* cnt = row_cursor + (int64_t)i * R;
    int32_t* rp = row_ptr + (int64_t)i * (R + 1);
    int carry = 0;
    for (int base = 0; base < R; base += kThreads) {
      const int r = base + tid;
      int part[kCounterCopies];
      int x = 0;
#pragma unroll
      for (int cpy = 0; cpy < kCounterCopies; ++cpy) {
        part[cpy] = r < R ? cnt[cpy * HR + r] : 0;
        x += part[cpy];
      }
      int tot;
      const int inc = block_inclusive_scan(x, s_warp, &tot);
      if (r < R) {
        rp[r + 1] = carry + inc;
        // the copies' fill cursors: consecutive sub-ranges of the row
        int start = carry + inc - x;
#pragma unroll
        for (int cpy = 0; cpy < kCounterCopies; ++cpy) {
          cnt[cpy * HR + r] = start;
          start += part[cpy];
        }
      }
      carry += tot;
    }
    if (tid == 0) { rp[0] = 0; head_off[i] = n_total; }
    n_total += carry;
  }
  if (tid == 0) {
    head_off[Hkv] = n_total;
    const int n = n_total;
    const int rpc = n < kRowsPerWalkSwitch ? kRowsPerWalkSmall : kRowsPerWalkLarge;
    const int full = n / rpc;
    const int tail = n - full * rpc;
    const int tail_walks = tail < num_cus ? tail : num_cus;
    desc[0] = n;
    desc[1] = rpc;
    desc[2] = full;
    desc[3] = tail;
    desc[4] = tail_walks;
    desc[5] = full + tail_walks;
    desc[6] = (int)cap;
    desc[7] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(
    int Hkv, int C, int K, int R, const int32_t* __restrict__ sel_clean,
    const int32_t* __restrict__ chunk_doc, const int32_t* __restrict__ doc_chunk_off,
    const int32_t* __restrict__ doc_blk_off, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ head_off, int32_t* __restrict__ row_cursor, int32_t* __restrict__ q_idx,
    int32_t* __restrict__ task_meta) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t cap1 = (int64_t)C * K;
  if (idx >= (int64_t)Hkv * cap1) return;
  int32_t* cursor = row_cursor + (int64_t)(blockIdx.x % kCounterCopies) * Hkv * R;
  const int i = (int)(idx / cap1);
  const int64_t e = idx - (int64_t)i * cap1;
  const int g = (int)(e / K);
  const int b = sel_clean[idx];
  if (b >= 0) {
    const int d = chunk_doc[g];
    const int c = g - doc_chunk_off[d];
    const int pos = atomicAdd(&cursor[(int64_t)i * R + doc_blk_off[d] + b], 1);
    q_idx[(int64_t)i * cap1 + pos] = kChunk * c;
  }
  if (e >= row_ptr[(int64_t)i * (R + 1) + R]) q_idx[idx] = -1;
  if (idx >= head_off[Hkv]) {
    int32_t* m = task_meta + idx * 6;
    for (int x = 0; x < 6; ++x) m[x] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void sort_kernel(
    const int32_t* __restrict__ cu, int Hkv, int C, int K, int R, int num_docs,
    const int32_t* __restrict__ doc_blk_off, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ head_off, int32_t* __restrict__ q_idx, int32_t* __restrict__ task_meta) {
  extern __shared__ uint32_t s_bits[];
  __shared__ int s_warp[kThreads / 64];
  const int i = blockIdx.x / R;
  const int r = blockIdx.x - i * R;
  const int tid = threadIdx.x;
  const int32_t* rp = row_ptr + (int64_t)i * (R + 1);
  const int lo = rp[r], n = rp[r + 1] - lo;
  if (n == 0) return;
  int d = upper_bound_minus1(doc_blk_off, num_docs + 1, r);
  d = d < num_docs ? d : num_docs - 1;
  const int b = r - doc_blk_off[d];
  const int len = cu[d + 1] - cu[d];
  const int nwords = ((len + kChunk - 1) / kChunk + 31) / 32;
  int32_t* qi = q_idx + (int64_t)i * C * K + lo;
  int32_t* meta = task_meta + ((int64_t)head_off[i] + lo) * 6;
  for (int w = tid; w < nwords; w += kThreads) s_bits[w] = 0;
  __syncthreads();
  for (int e = tid; e < n; e += kThreads) {
    const int c = qi[e] / kChunk;
    atomicOr(&s_bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // Each thread owns a contiguous run of words; ranks come from a block scan.
  const int per = (nwords + kThreads - 1) / kThreads;
  const int w0 = tid * per, w1 = min(nwords, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(s_bits[w]);
  int tot;
  int rank = block_inclusive_scan(cnt, s_warp, &tot) - cnt;
  for (int w = w0; w < w1; ++w) {
    uint32_t word = s_bits[w];
    while (word) {
      const int bit = __ffs(word) - 1;
      word &= word - 1;
      const int q0 = kChunk * (32 * w + bit);
      qi[rank] = q0;
      int32_t* m = meta + (int64_t)rank * 6;
      m[0] = i;
      m[1] = r;
      m[2] = q0;
      m[3] = min(kChunk, len - q0);
      m[4] = d;
      m[5] = b;
      ++rank;
    }
  }
}

}  // namespace

hipError_t launch_build_schedule(const msa_problem& p, const int32_t* cu, const int32_t* sel,
                                 const int32_t* kv_starts, int32_t* sched, const msa_schedule_layout& L,
                                 hipStream_t stream) {
  const int Hkv = p.num_kv_heads, C = p.num_chunks, K = p.topk, R = p.num_kblocks;
  const int64_t cap = (int64_t)Hkv * C * K;
  // clean and fill must use the same grid: a slot's counter copy is its
  // workgroup id modulo kCounterCopies in both
  const int64_t n_cursor = (int64_t)kCounterCopies * Hkv * R;
  const unsigned zero_blocks = (unsigned)((n_cursor + kZeroPerBlock - 1) / kZeroPerBlock);
  hipLaunchKernelGGL(geometry_kernel, dim3(1 + zero_blocks), dim3(kThreads), 0, stream, cu, kv_starts,
                     p.num_docs, p.total_tokens, (int)kv_rows_of(p), C, R, p.block_size, p.max_doc_chunks,
                     sched + L.doc_chunk_off, sched + L.doc_blk_off, sched + L.doc_kv_off, sched + L.desc,
                     sched + L.err, sched + L.row_cursor, n_cursor);
  const unsigned grid = (unsigned)((cap + kThreads - 1) / kThreads);
  if (cap > 0)
    hipLaunchKernelGGL(clean_kernel, dim3(grid), dim3(kThreads), 0, stream, cu, sel, Hkv, C, K, R, p.block_size,
                       p.num_docs, sched + L.doc_chunk_off, sched + L.doc_blk_off, sched + L.chunk_doc,
                       sched + L.sel_clean, sched + L.row_cursor, sched + L.err);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kThreads), 0, stream, Hkv, R, cap, p.num_cus,
                     sched + L.row_cursor, sched + L.row_ptr, sched + L.head_off, sched + L.desc);
  if (cap > 0)
    hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(kThreads), 0, stream, Hkv, C, K, R,
                       sched + L.sel_clean, sched + L.chunk_doc, sched + L.doc_chunk_off,
                       sched + L.doc_blk_off, sched + L.row_ptr, sched + L.head_off,
                       sched + L.row_cursor, sched + L.q_idx, sched + L.task_meta);
  if ((int64_t)Hkv * R > 0) {
    const size_t lds = sizeof(uint32_t) * (size_t)((p.max_doc_chunks + 31) / 32);
    hipLaunchKernelGGL(sort_kernel, dim3((unsigned)(Hkv * R)), dim3(kThreads), lds, stream, cu, Hkv, C,
                       K, R, p.num_docs, sched + L.doc_blk_off, sched + L.row_ptr, sched + L.head_off,
                       sched + L.q_idx, sched + L.task_meta);
  }
  return hipGetLastError();
}

}  // namespace msa
