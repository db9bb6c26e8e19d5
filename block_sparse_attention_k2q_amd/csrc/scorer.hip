// Index scorer and top-k block selection (gfx950): the step that produces
// the block selection the sparse attention consumes.
//
// The pages name the scorer (msa_bindings page: MSAKernels lists
// fmha_sm100, "the scorer", beside the planner) and give its sizes
// (msa_schedule page, module data: INDEX_DIM 128, NUM_INDEX_HEADS 4,
// TOPK_BLOCKS 16) but not the scoring function.  This library's reading,
// per index head i:
//   score(c, b) = (sum of the index queries of chunk c)
//                 . (mean of the index keys of key block b),
// over the tokens of the chunk's document; the chunk keeps its own
// (diagonal) block and the topk - 1 best-scoring earlier blocks of the
// document (ties to the smaller block id, fewer when fewer exist), written
// ascending with -1 padding -- the selection format msa_build_schedule reads.
//
// Kernels, all on one stream:
//   geometry   one workgroup: per-document chunk / block offsets from
//              cu_seqlens, checked against the host sizes (a mismatch makes
//              every selection row empty);
//   pool       one wave per (head, key block) and per (head, chunk): fp32
//              block key means and chunk query sums, tokens summed in order;
//   select     one wave per (head, chunk): the scores of the chunk's earlier
//              blocks (16 lanes per block, 8 dimensions each, then a 16-lane
//              tree) into LDS, then topk - 1 rounds of a wave argmax.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / 64;

__global__ __launch_bounds__(kIdxThreads) void index_geometry_kernel(
    const int32_t* __restrict__ cu, int num_docs, int T, int C, int R, int B, int max_doc_chunks,
    int32_t* __restrict__ doc_chunk_off, int32_t* __restrict__ doc_blk_off, int32_t* __restrict__ err) {
  __shared__ int s_warp[kIdxWaves];
  const int tid = threadIdx.x;
  int bad = 0, carry_c = 0, carry_b = 0;
  for (int base = 0; base < num_docs; base += kIdxThreads) {
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
    }
    int tc, tb;
    const int ic = block_inclusive_scan_n<kIdxThreads>(nc, s_warp, &tc);
    const int ib = block_inclusive_scan_n<kIdxThreads>(nb, s_warp, &tb);
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
  if (tid == 0) err[0] = bad;
}

// Unit u < H*R: block key mean of (head u / R, row u % R); else chunk query
// sum of (head, chunk) = divmod(u - H*R, C).  Lane l owns dimensions 2l, 2l+1.
__global__ __launch_bounds__(kIdxThreads) void index_pool_kernel(
    const bf16* __restrict__ qi, const bf16* __restrict__ ki, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ doc_blk_off,
    const int32_t* __restrict__ err, int H, int C, int R, int B, int num_docs, float* __restrict__ qsum,
    float* __restrict__ kbar) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int64_t u = (int64_t)blockIdx.x * kIdxWaves + wave_id();
  const int lane = lane_id();
  const int64_t HR = (int64_t)H * R;
  if (u >= HR + (int64_t)H * C || err[0]) return;
  const bool is_key = u < HR;
  const int64_t v = is_key ? u : u - HR;
  const int n_rows = is_key ? R : C;
  const int i = (int)(v / n_rows), r = (int)(v - (int64_t)i * n_rows);
  const int32_t* off = is_key ? doc_blk_off : doc_chunk_off;
  int d = upper_bound_minus1(off, num_docs + 1, r);
  d = d < num_docs ? d : num_docs - 1;
  const int tok0 = cu[d], len = cu[d + 1] - tok0;
  const int span = is_key ? B : kChunk;
  const int first = (r - off[d]) * span;
  const int count = min(span, len - first);
  const bf16* src = (is_key ? ki : qi) + ((int64_t)(tok0 + first) * H + i) * kIndexDim + 2 * lane;
  float a0 = 0.f, a1 = 0.f;
  const int64_t stride = (int64_t)H * kIndexDim;
  int t = 0;
  for (; t + 4 <= count; t += 4) {   // four loads in flight, then added in token order
    bf16x2 x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) x[m] = *reinterpret_cast<const bf16x2*>(src + (t + m) * stride);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      a0 += (float)x[m][0];
      a1 += (float)x[m][1];
    }
  }
  for (; t < count; ++t) {
    const bf16x2 x = *reinterpret_cast<const bf16x2*>(src + t * stride);
    a0 += (float)x[0];
    a1 += (float)x[1];
  }
  if (is_key) {
    a0 /= (float)count;
    a1 /= (float)count;
  }
  float* dst = (is_key ? kbar : qsum) + v * kIndexDim + 2 * lane;
  *reinterpret_cast<float2*>(dst) = make_float2(a0, a1);
}

// (score, id) order of the selection: higher score first, then smaller id.
__device__ __forceinline__ bool better(float s, int b, float s2, int b2) {
  return s > s2 || (s == s2 && b < b2);
}

__global__ __launch_bounds__(kIdxThreads) void index_select_kernel(
    const float* __restrict__ qsum, const float* __restrict__ kbar, const int32_t* __restrict__ doc_chunk_off,
    const int32_t* __restrict__ doc_blk_off, const int32_t* __restrict__ err, int H, int C, int R, int B,
    int K, int num_docs, int cand_cap, int32_t* __restrict__ sel) {
  // cand_cap floats of scores per wave (the longest document's block count,
  // at most kMaxIndexCandidates), sized at launch
  extern __shared__ float s_score[];
  const int w = wave_id(), lane = lane_id();
  const int64_t unit = (int64_t)blockIdx.x * kIdxWaves + w;   // = i * C + g
  if (unit >= (int64_t)H * C) return;   // whole waves; the kernel has no workgroup barrier
  int32_t* out = sel + unit * K;
  if (err[0]) {
    for (int s = lane; s < K; s += 64) out[s] = -1;
    return;
  }
  const int i = (int)(unit / C), g = (int)(unit - (int64_t)i * C);
  int d = upper_bound_minus1(doc_chunk_off, num_docs + 1, g);
  d = d < num_docs ? d : num_docs - 1;
  const int c = g - doc_chunk_off[d];
  const int diag = (kChunk * c) / B;   // candidates: blocks 0 .. diag - 1
  const int n = diag;
  float* sc = s_score + w * cand_cap;

  // Scores: lane group grp = lane / 16 takes block b0 + grp; lane sl = lane % 16
  // of the group multiplies dimensions 8 sl .. 8 sl + 7 in order, then the
  // group adds its 16 partial sums pairwise (xor 8, 4, 2, 1).
  const int grp = lane >> 4, sl = lane & 15;
  const float4* qv = reinterpret_cast<const float4*>(qsum + unit * kIndexDim + 8 * sl);
  const float4 q0 = qv[0], q1 = qv[1];
  const float* krows = kbar + ((int64_t)i * R + doc_blk_off[d]) * kIndexDim + 8 * sl;
  // Four blocks per group per round, their loads issued together.
  constexpr int kRound = 4;
  for (int b0 = 0; b0 < n; b0 += 4 * kRound) {
    float4 k0[kRound], k1[kRound];
#pragma unroll
    for (int t = 0; t < kRound; ++t) {
      const int b = b0 + 4 * t + grp;
      if (b < n) {
        const float4* kv = reinterpret_cast<const float4*>(krows + (int64_t)b * kIndexDim);
        k0[t] = kv[0];
        k1[t] = kv[1];
      } else {
        k0[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        k1[t] = k0[t];
      }
    }
#pragma unroll
    for (int t = 0; t < kRound; ++t) {
      const int b = b0 + 4 * t + grp;
      float part = q0.x * k0[t].x;
      part = fmaf(q0.y, k0[t].y, part);
      part = fmaf(q0.z, k0[t].z, part);
      part = fmaf(q0.w, k0[t].w, part);
      part = fmaf(q1.x, k1[t].x, part);
      part = fmaf(q1.y, k1[t].y, part);
      part = fmaf(q1.z, k1[t].z, part);
      part = fmaf(q1.w, k1[t].w, part);
      part += __shfl_xor(part, 8, 64);
      part += __shfl_xor(part, 4, 64);
      part += __shfl_xor(part, 2, 64);
      part += __shfl_xor(part, 1, 64);
      if (b < n && sl == 0) sc[b] = part;
    }
  }
  wave_lds_sync();   // the wave's score writes before its reads

  // topk - 1 rounds of a wave argmax; lane l owns candidates l, l + 64, ...
  const int m = min(K - 1, n);
  int mine = INT32_MAX;   // lane r < m: the block chosen in round r
  if (n <= K - 1) {
    mine = lane < n ? lane : INT32_MAX;
  } else {
    float best_s = -INFINITY;
    int best_b = INT32_MAX;
    auto rescan = [&]() {
      best_s = -INFINITY;
      best_b = INT32_MAX;
      for (int b = lane; b < n; b += 64) {
        const float s = sc[b];
        if (better(s, b, best_s, best_b)) { best_s = s; best_b = b; }
      }
    };
    rescan();
    for (int round = 0; round < m; ++round) {
      float s = best_s;
      int b = best_b;
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) {
        const float s2 = __shfl_xor(s, x, 64);
        const int b2 = __shfl_xor(b, x, 64);
        if (better(s2, b2, s, b)) { s = s2; b = b2; }
      }
      if (lane == round) mine = b;
      if ((b & 63) == lane) {
        sc[b] = -INFINITY;
        wave_lds_sync();
        rescan();
      }
    }
  }
  // the diagonal block joins in slot m; write the m + 1 ids ascending
  if (lane == m) mine = diag;
  const int count = m + 1;
  int rank = 0;
  for (int t = 0; t < count; ++t) rank += __shfl(mine, t, 64) < mine;
  if (lane < count) out[rank] = mine;
  for (int s = count + lane; s < K; s += 64) out[s] = -1;
}

}  // namespace

hipError_t launch_index_select(const msa_problem& p, const void* qi, const void* ki, const int32_t* cu,
                               void* scratch, int32_t* sel, hipStream_t stream) {
  const IndexScratch S = index_scratch_layout(p);
  uint8_t* base = (uint8_t*)scratch;
  int32_t* geo = (int32_t*)(base + S.geo);
  int32_t* doc_chunk_off = geo;
  int32_t* doc_blk_off = geo + p.num_docs + 1;
  int32_t* err = doc_blk_off + p.num_docs + 1;
  float* qsum = (float*)(base + S.qsum);
  float* kbar = (float*)(base + S.kbar);
  const int H = p.num_kv_heads, C = p.num_chunks, R = p.num_kblocks, B = p.block_size;
  hipLaunchKernelGGL(index_geometry_kernel, dim3(1), dim3(kIdxThreads), 0, stream, cu, p.num_docs,
                     p.total_tokens, C, R, B, p.max_doc_chunks, doc_chunk_off, doc_blk_off, err);
  const int64_t pool_units = (int64_t)H * (R + C);
  if (pool_units > 0)
    hipLaunchKernelGGL(index_pool_kernel, dim3((unsigned)((pool_units + kIdxWaves - 1) / kIdxWaves)),
                       dim3(kIdxThreads), 0, stream, (const bf16*)qi, (const bf16*)ki, cu, doc_chunk_off,
                       doc_blk_off, err, H, C, R, B, p.num_docs, qsum, kbar);
  const int64_t sel_units = (int64_t)H * C;
  // candidates of a chunk: the earlier blocks of its document
  const int64_t max_doc_blocks = ((int64_t)p.max_doc_chunks * kChunk + B - 1) / B;
  const int cand_cap = (int)((max_doc_blocks + 63) / 64 * 64);
  if (sel_units > 0)
    hipLaunchKernelGGL(index_select_kernel, dim3((unsigned)((sel_units + kIdxWaves - 1) / kIdxWaves)),
                       dim3(kIdxThreads), (size_t)kIdxWaves * cand_cap * sizeof(float), stream, qsum, kbar,
                       doc_chunk_off, doc_blk_off, err, H, C, R, B, p.topk, p.num_docs, cand_cap, sel);
  return hipGetLastError();
}

}  // namespace msa
