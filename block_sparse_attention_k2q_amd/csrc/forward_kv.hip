// Planner-driven (KV-parallel) forward of MSA main attention on gfx950.
//
// The pages list a planner beside the flat forward (msa_bindings: MSAKernels,
// fmha_sm100_plan) whose work items are the rows of scheduler_metadata
// (msa_schedule page: MSABackwardSchedule, one item per k2q CSR entry).  This
// forward walks those items the way the KV-parallel backward does: each
// workgroup takes a walk of task rows, holds the key block of the current
// bucket in LDS and brings in the 128 query rows of each task.  The rows of
// one chunk are then spread over as many workgroups as the chunk has blocks,
// so the softmax has to be reduced across workgroups.  It is done exactly, in
// four launches:
//   stats   per task and query row: m = the row's largest scaled score in
//           the block (log2 domain) and l = sum exp2(s - m) over its keys,
//           fp32, into a slot per (index head, chunk, selection slot);
//   merge   per query row: LSE = M + log2(sum_t l_t 2^(m_t - M)) over the
//           chunk's slots (natural-log lse written), and the row of an fp32
//           output pool cleared;
//   output  per task again: P = exp2(s - LSE) (the final probabilities, split
//           into bf16 high and low parts so the weights are fp32-accurate),
//           O = P V for the task's 128 rows, added into the pool with fp32
//           atomics;
//   cast    out = bf16(pool).
// It computes S twice and adds O with atomics, which is what spreading a
// chunk over workgroups costs on this chip (the query-parallel forward of
// forward.hip keeps a chunk's online softmax in one workgroup instead).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kFkvThreads = 256;   // 4 waves, 32 query rows each
constexpr int kFkvMaxWalk = 64;    // ROWS_PER_CTA_LARGE

template <int D>
struct FkvSmem {
  static constexpr int LDK = D + 8;   // padded rows
  bf16 k[kBlock * LDK];
  bf16 v[kBlock * LDK];
  bf16 q[kTileM * LDK];
  float lse2[kTileM];                 // output pass: LSE * log2(e) per row, +inf past the end
  int meta[kFkvMaxWalk][9];           // i, r, qb, qc, slot, b, tok0, len, kv0
};

// PASS 0: statistics; PASS 1: output.
template <int D, int PASS>
__global__ __launch_bounds__(kFkvThreads, 2) void forward_kv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ task_meta, const int32_t* __restrict__ desc,
    const int32_t* __restrict__ err, const int32_t* __restrict__ doc_chunk_off,
    const int32_t* __restrict__ doc_kv_off, const int32_t* __restrict__ sel_clean,
    float2* __restrict__ stats, const float* __restrict__ lse, float* __restrict__ pool, int Hkv, int C,
    int K, float scale) {
  using S = FkvSmem<D>;
  constexpr int LDK = S::LDK;
  constexpr int KS = D / 16;
  constexpr int NT = D / 32;
  constexpr int VEC = D / 8;
  __shared__ __attribute__((aligned(16))) S sm;

  if (err[1]) return;
  const int wg = blockIdx.x;
  if (wg >= desc[5]) return;
  const int rpc = desc[1], full = desc[2], tail = desc[3], tail_walks = desc[4];
  int lo, hi;
  if (wg < full) {
    lo = wg * rpc;
    hi = lo + rpc;
  } else {
    const int t = wg - full;
    const int base = tail / tail_walks, extra = tail % tail_walks;
    lo = full * rpc + t * base + min(t, extra);
    hi = lo + base + (t < extra ? 1 : 0);
  }
  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;
  const int Hq = Hkv * kQPerKV;
  const float c2 = scale * kLog2e;
  const int mq = 32 * w + n32;          // this lane's query row (token mq / 16, head mq % 16)

  const int nrows = hi - lo;
  for (int e = threadIdx.x; e < nrows; e += kFkvThreads) {
    const int32_t* tm = task_meta + (int64_t)(lo + e) * 6;
    int* m = sm.meta[e];
#pragma unroll
    for (int x = 0; x < 6; ++x) m[x] = tm[x];
    const int d = tm[4];
    const int t0 = cu[d];
    m[6] = t0;
    m[7] = cu[d + 1] - t0;
    m[8] = doc_kv_off[d];
    // the task's slot: (index head, global chunk, position of its block in
    // the chunk's cleaned selection)
    const int64_t row = (int64_t)tm[0] * C + doc_chunk_off[d] + tm[2] / kChunk;
    int slot = -1;
    for (int x = 0; x < K; ++x) slot = sel_clean[row * K + x] == tm[5] ? x : slot;
    m[4] = slot < 0 ? -1 : (int)(row * K + slot);
  }
  lds_barrier();

  int cur_i = -1, cur_r = -1;
  for (int e = 0; e < nrows; ++e) {
    const int* mrow = sm.meta[e];
    const int i = mrow[0], r = mrow[1], qb = mrow[2], qc = mrow[3], slot = mrow[4], b = mrow[5];
    const int tok0 = mrow[6], len = mrow[7], kv0 = mrow[8];
    lds_barrier();   // every wave is done with the previous task's tiles
    if (i != cur_i || r != cur_r) {
      cur_i = i;
      cur_r = r;
      // K and V of the block; keys past the document end read its last key
      // (they are masked)
      for (int x = threadIdx.x; x < kBlock * VEC; x += kFkvThreads) {
        const int kr = x / VEC, col = (x % VEC) * 8;
        const int64_t off = ((int64_t)(kv0 + min(b * kBlock + kr, len - 1)) * Hkv + i) * D + col;
        *reinterpret_cast<u32x4*>(&sm.k[kr * LDK + col]) = *reinterpret_cast<const u32x4*>(k + off);
        if constexpr (PASS == 1)
          *reinterpret_cast<u32x4*>(&sm.v[kr * LDK + col]) = *reinterpret_cast<const u32x4*>(v + off);
      }
    }
    // the task's 128 query rows; rows past the document end repeat its last token
    for (int x = threadIdx.x; x < kTileM * VEC; x += kFkvThreads) {
      const int mm = x / VEC, col = (x % VEC) * 8;
      const int j = min(mm >> 4, qc - 1);
      const int64_t off = ((int64_t)(tok0 + qb + j) * Hq + kQPerKV * i + (mm & 15)) * D + col;
      *reinterpret_cast<u32x4*>(&sm.q[mm * LDK + col]) = *reinterpret_cast<const u32x4*>(q + off);
    }
    if constexpr (PASS == 1) {
      if (threadIdx.x < kTileM) {
        const int mm = threadIdx.x;
        const int j = mm >> 4;
        const float l = j < qc ? lse[(int64_t)(tok0 + qb + j) * Hq + kQPerKV * i + (mm & 15)] : -INFINITY;
        sm.lse2[mm] = l == -INFINITY ? INFINITY : l * kLog2e;   // P = 0 for rows that see no key
      }
    }
    lds_barrier();

    // S^T = K Q^T for this wave's 32 query columns: two 32-key tiles
    floatx16 st[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 bq = load_bf16x8_lds(&sm.q[mq * LDK + 16 * s + 8 * h]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        st[t] = mfma32(load_bf16x8_lds(&sm.k[(32 * t + n32) * LDK + 16 * s + 8 * h]), bq, st[t]);
    }
    // causal and document-end mask (only the diagonal block has keys after a
    // query or past the end); key offset of register j of tile t:
    // 32t + 8(j/4) + 4h + j%4
    const int jtok = mq >> 4;
    const bool valid = jtok < qc;
    if ((b + 1) * kBlock - 1 > qb) {
      const int klim = min(qb + jtok, len - 1) - b * kBlock - 4 * h;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) st[t][j] = 32 * t + 8 * (j >> 2) + (j & 3) <= klim ? st[t][j] : -INFINITY;
    }

    if constexpr (PASS == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[t][j]);
      {
        const auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1])) * c2;
      }
      float l = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 16; ++j) l += fast_exp2(fmaf(st[t][j], c2, -mx));
      }
      {
        const auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
        l = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
      }
      if (h == 0 && slot >= 0)
        stats[(int64_t)slot * kTileM + mq] = valid ? make_float2(mx, l) : make_float2(-INFINITY, 0.f);
    } else {
      const float l2 = sm.lse2[mq];
      // P in k steps of 16 keys (registers 8(u%2) .. +7 of tile u/2), as bf16
      // high and low parts
      bf16x8 ph[4], pl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p = fast_exp2(fmaf(st[u >> 1][8 * (u & 1) + x], c2, -l2));
          ph[u][x] = (bf16)p;
          pl[u][x] = (bf16)(p - (float)ph[u][x]);
        }
      // O (32 query rows x D) = P V: P straight from the S^T registers (the
      // contraction runs over keys, their row index), V through the transpose load
      floatx16 o[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] = floatx16{};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 bv = lds_tr_operand(sm.v, LDK, 32 * t, lane, 16 * u, 16 * u + 4, 16 * u + 8, 16 * u + 12);
          o[t] = mfma32(ph[u], bv, o[t]);
          o[t] = mfma32(pl[u], bv, o[t]);
        }
      // register j of d tile t: query row 32w + 8(j/4) + 4h + j%4, dim 32t + n32;
      // rows past the document end hold exact zeros and go to the tile's first row
      const int64_t row0 = (int64_t)(tok0 + qb) * Hq + kQPerKV * i;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
        const int jt = m >> 4;
        const int64_t rowm = jt < qc ? row0 + (int64_t)jt * Hq + (m & 15) : row0;
        float* dst = pool + rowm * D + n32;
#pragma unroll
        for (int t = 0; t < NT; ++t) atomicAdd(dst + 32 * t, o[t][j]);
      }
    }
  }
}

// One thread per query row of an (index head, chunk): merge the chunk's slots
// into the row's LSE and clear its row of the output pool.
template <int D>
__global__ __launch_bounds__(kTileM) void forward_kv_merge_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ sel_clean,
    const int32_t* __restrict__ err, const float2* __restrict__ stats, float* __restrict__ lse,
    float* __restrict__ pool, int Hkv, int C, int K) {
  if (err[1]) return;
  const int i = blockIdx.x % Hkv;
  const int g = blockIdx.x / Hkv;
  const int d = chunk_doc[g];
  const int c = g - doc_chunk_off[d];
  const int tok0 = cu[d];
  const int qcount = min(kChunk, cu[d + 1] - tok0 - kChunk * c);
  const int mm = threadIdx.x;
  if ((mm >> 4) >= qcount) return;
  const int Hq = Hkv * kQPerKV;
  const int64_t rowi = (int64_t)(tok0 + kChunk * c + (mm >> 4)) * Hq + kQPerKV * i + (mm & 15);
  const int64_t sel0 = ((int64_t)i * C + g) * K;
  float M = -INFINITY;
  for (int s = 0; s < K; ++s)
    if (sel_clean[sel0 + s] >= 0) M = fmaxf(M, stats[(sel0 + s) * kTileM + mm].x);
  float L = 0.f;
  if (M != -INFINITY)
    for (int s = 0; s < K; ++s)
      if (sel_clean[sel0 + s] >= 0) {
        const float2 st = stats[(sel0 + s) * kTileM + mm];
        if (st.y > 0.f) L += st.y * fast_exp2(st.x - M);
      }
  lse[rowi] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
  floatx4* pr = reinterpret_cast<floatx4*>(pool + rowi * D);
#pragma unroll
  for (int x = 0; x < D / 4; ++x) pr[x] = floatx4{};
}

__global__ __launch_bounds__(256) void forward_kv_cast_kernel(const float* __restrict__ pool,
                                                              bf16* __restrict__ out, int64_t n_vec,
                                                              float* __restrict__ lse, int64_t n_lse,
                                                              const int32_t* __restrict__ err) {
  if (err[1]) {   // geometry mismatch: the passes before did not run
    fill_nan(out, n_vec, lse, n_lse);
    return;
  }
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n_vec) return;
  const floatx4 a = reinterpret_cast<const floatx4*>(pool)[2 * x];
  const floatx4 b = reinterpret_cast<const floatx4*>(pool)[2 * x + 1];
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)a[e];
    r[4 + e] = (bf16)b[e];
  }
  store_bf16x8(out + 8 * x, r);
}

}  // namespace

hipError_t launch_forward_kv(const msa_problem& p, const void* q, const void* k, const void* v,
                             const int32_t* cu, const int32_t* sched, const msa_schedule_layout& L,
                             void* scratch, void* out, float* lse, hipStream_t stream) {
  const ForwardKvScratch S = forward_kv_scratch_layout(p);
  uint8_t* base = (uint8_t*)scratch;
  float2* stats = (float2*)(base + S.stats);
  float* pool = (float*)(base + S.pool);
  const int64_t nwg = (int64_t)p.num_chunks * p.num_kv_heads;
  if (nwg == 0) return hipSuccess;
  const int64_t cap = (int64_t)p.num_kv_heads * p.num_chunks * p.topk;
  const int64_t grid = grid_launch_bound(cap, p.num_cus);
  auto walk = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kFkvThreads), 0, stream, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, cu, sched + L.task_meta, sched + L.desc, sched + L.err,
                       sched + L.doc_chunk_off, sched + L.doc_kv_off, sched + L.sel_clean, stats, lse, pool,
                       p.num_kv_heads, p.num_chunks, p.topk, p.softmax_scale);
  };
  auto merge = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kTileM), 0, stream, cu, sched + L.chunk_doc,
                       sched + L.doc_chunk_off, sched + L.sel_clean, sched + L.err, stats, lse, pool,
                       p.num_kv_heads, p.num_chunks, p.topk);
  };
  if (p.head_dim == 128) {
    walk(forward_kv_kernel<128, 0>);
    merge(forward_kv_merge_kernel<128>);
    walk(forward_kv_kernel<128, 1>);
  } else {
    walk(forward_kv_kernel<64, 0>);
    merge(forward_kv_merge_kernel<64>);
    walk(forward_kv_kernel<64, 1>);
  }
  const int64_t n_vec = (int64_t)p.total_tokens * p.num_kv_heads * kQPerKV * p.head_dim / 8;
  if (n_vec > 0)
    hipLaunchKernelGGL(forward_kv_cast_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256), 0, stream,
                       (const float*)pool, (bf16*)out, n_vec, lse,
                       (int64_t)p.total_tokens * p.num_kv_heads * kQPerKV, sched + L.err);
  return hipGetLastError();
}

}  // namespace msa
