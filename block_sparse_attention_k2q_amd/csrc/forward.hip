// Sparse forward of MSA main attention on gfx950.
//
// The pages name the flat forward (msa_bindings: sparse_atten_func) and fix
// what it must hand the backward (msa_backward_sm100: run_backward takes the
// forward's bf16 out [T, Hq, D] and fp32 lse [T, Hq]).  The kernel below is
// this library's own design for CDNA4:
//
//  * one workgroup of 2 waves per (chunk, index head): a 128-row query tile
//    of 8 tokens x 16 query heads sharing one KV head, each wave owning 64
//    rows (two 32-query MFMA columns).  Workgroup ids run head-fastest, so
//    with 4 or 8 KV heads each XCD (ids are dealt to the 8 XCDs round-robin)
//    reads the K/V of one head only, which then stays in its L2;
//  * the tile's Q rows live in registers as MFMA B operands for the whole
//    chunk;
//  * per kept key block (64 keys): K and V arrive in LDS by direct
//    global->LDS loads into one of two swizzled buffers, the next block's
//    copy in flight while the current one is consumed (one barrier per
//    block);  S^T = K Q^T (keys x queries, so a lane owns one query column),
//    online softmax in the exp2 domain with the causal mask, and
//    O^T += V^T P^T with P^T taken straight from the S^T accumulators and V^T
//    read by the LDS transpose load;
//  * out = O / l in bf16, lse = ln(sum exp(scale * s)) in fp32.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr float kRescaleLog2 = 8.f;
// One 32-query column per wave (4 waves per tile) fits 256 registers, so two
// waves share each SIMD; two columns per wave halve the LDS reads but need
// ~300 registers (one wave per SIMD) and measured slower.
constexpr int kFwdNQ = 1;

// NQ = 32-query MFMA columns per wave; the 128-row tile takes 4 / NQ waves.
template <int D, int NQ>
__global__ __launch_bounds__(256 / NQ, NQ == 1 ? 2 : 1) void forward_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ sel_clean,
    const int32_t* __restrict__ err, bf16* __restrict__ out, float* __restrict__ lse, int Hkv, int C,
    int K, float scale) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;           // k steps of S^T = K Q^T
  constexpr int NT = D / 32;           // 32-wide d tiles of O^T
  constexpr int NW = 4 / NQ;            // waves per workgroup
  __shared__ __attribute__((aligned(16))) KVTiles<D> buf0;
  __shared__ __attribute__((aligned(16))) KVTiles<D> buf1;
  __shared__ int s_blocks[64];
  __shared__ int s_nblocks;

  if (err[1]) return;
  const int i = blockIdx.x % Hkv;
  const int g = blockIdx.x / Hkv;
  const int d = chunk_doc[g];
  const int c = g - doc_chunk_off[d];
  const int tok0 = cu[d];
  const int len = cu[d + 1] - tok0;
  const int p0 = kChunk * c;
  const int qcount = min(kChunk, len - p0);
  const int Hq = Hkv * kQPerKV;

  if (threadIdx.x < 64) {
    const int n = compact_selection(sel_clean + ((int64_t)i * C + g) * K, K, threadIdx.x, s_blocks, nullptr);
    if (threadIdx.x == 0) s_nblocks = n;
  }

  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;
  // Query column nq of this lane: tile row 32(NQ w + nq) + n32, i.e. token
  // 2(NQ w + nq) + n32/16 and head n32%16.
  int jq[NQ], pq[NQ];
  bool qvalid[NQ];
  int64_t qrow[NQ];
  bf16x8 qf[NQ][KS];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    jq[nq] = 2 * (NQ * w + nq) + (n32 >> 4);
    qvalid[nq] = jq[nq] < qcount;
    pq[nq] = p0 + jq[nq];
    qrow[nq] = (int64_t)(tok0 + p0 + min(jq[nq], qcount - 1)) * Hq + kQPerKV * i + (n32 & 15);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[nq][s] = qvalid[nq] ? load_bf16x8(q + qrow[nq] * D + 16 * s + 8 * h) : bf16x8{};
  }

  floatx16 o[NT][NQ];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) o[t][nq] = floatx16{};
  float m[NQ], l[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) { m[nq] = -INFINITY; l[nq] = 0.f; }
  const float c2 = scale * kLog2e;

  lds_barrier();
  const int nblk = s_nblocks;
  const KvCopier<D, NW> copy_kv(Hkv, w, lane);
  if (nblk > 0) copy_kv(buf0, k, v, tok0, len, s_blocks[0], i);

  auto consume = [&](const KVTiles<D>& t, int b) {
    // S^T = K Q^T: two 32-key tiles x two query columns; operands of k step
    // s+1 are read while step s runs.
    floatx16 st[2][NQ];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) st[a][nq] = floatx16{};
    bf16x8 ak[2][2];
    ak[0][0] = lds_row8<CPR>(t.k, n32, 8 * h);
    ak[0][1] = lds_row8<CPR>(t.k, 32 + n32, 8 * h);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) {
        ak[(s + 1) & 1][0] = lds_row8<CPR>(t.k, n32, 16 * (s + 1) + 8 * h);
        ak[(s + 1) & 1][1] = lds_row8<CPR>(t.k, 32 + n32, 16 * (s + 1) + 8 * h);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) st[a][nq] = mfma32(ak[s & 1][a], qf[nq][s], st[a][nq]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Online softmax per query column.  Only the diagonal block holds keys
    // after a query (or past the document end): there, keys at block offset
    // > klim are set to -inf before the max.
    const bool diag = (b + 1) * kBlock - 1 > p0;
    bf16x8 pb[NQ][4];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      if (diag) {
        const int klim = min(pq[nq], len - 1) - b * kBlock;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = 32 * a + 8 * (j >> 2) + 4 * h + (j & 3);
            st[a][nq][j] = key <= klim ? st[a][nq][j] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[a][nq][j]);
      mx = fmaxf(mx, swap_halves(mx)) * c2;   // max in the scaled log2 domain
      // Lazy rescale: the running max m only moves when a score exceeds it by
      // more than kRescaleLog2, so P = exp2(s - m) stays <= 2^kRescaleLog2 and
      // the O accumulators are rescaled only on the (rare) blocks that move it.
      const bool move = mx > m[nq] + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float m_new = move ? mx : m[nq];
        const float alpha = (m[nq] == -INFINITY) ? 0.f : fast_exp2(m[nq] - m_new);
        l[nq] *= alpha;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) o[tt][nq] *= alpha;
        m[nq] = m_new;
      }
      const float msub = (m[nq] == -INFINITY) ? 0.f : m[nq];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          pb[nq][2 * a + (j >> 3)][j & 7] = (bf16)fast_exp2(fmaf(st[a][nq][j], c2, -msub));
      // Row sum of the bf16 probabilities that enter O (same values normalise it).
#pragma unroll
      for (int u = 0; u < 4; ++u) l[nq] = sum_bf16x8(pb[nq][u], l[nq]);
    }

    // O^T += V^T P^T over 4 k steps of 16 keys; V^T operands double-buffered.
    bf16x8 av[2][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      av[0][tt] = lds_tr_operand_swz<CPR>(t.v, 32 * tt, lane, 0, 4, 8, 12);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u + 1 < 4) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          av[(u + 1) & 1][tt] = lds_tr_operand_swz<CPR>(t.v, 32 * tt, lane, 16 * (u + 1),
                                                        16 * (u + 1) + 4, 16 * (u + 1) + 8,
                                                        16 * (u + 1) + 12);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) o[tt][nq] = mfma32(av[u & 1][tt], pb[nq][u], o[tt][nq]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int bi = 0; bi < nblk; bi += 2) {
    // Even blocks use buf0, odd blocks buf1.
    wait_vmem();
    lds_barrier();   // block bi landed in buf0; all waves are done with buf1
    if (bi + 1 < nblk) copy_kv(buf1, k, v, tok0, len, s_blocks[bi + 1], i);
    consume(buf0, s_blocks[bi]);
    if (bi + 1 < nblk) {
      wait_vmem();
      lds_barrier();  // block bi+1 landed in buf1; all waves are done with buf0
      if (bi + 2 < nblk) copy_kv(buf0, k, v, tok0, len, s_blocks[bi + 2], i);
      consume(buf1, s_blocks[bi + 1]);
    }
  }

#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const float l_tot = l[nq] + swap_halves(l[nq]);
    if (!qvalid[nq]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* orow = out + qrow[nq] * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4 v4;
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = (bf16)(o[tt][nq][4 * jg + r] * inv);
        store_bf16x4(orow + 32 * tt + 8 * jg + 4 * h, v4);
      }
    }
    if (h == 0) lse[qrow[nq]] = l_tot > 0.f ? (m[nq] + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_forward(const msa_problem& p, const void* q, const void* k, const void* v,
                          const int32_t* cu, const int32_t* sched, const msa_schedule_layout& L,
                          void* out, float* lse, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_chunks * p.num_kv_heads;
  if (nwg == 0) return hipSuccess;
  auto args = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(threads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, cu, sched + L.chunk_doc, sched + L.doc_chunk_off,
                       sched + L.sel_clean, sched + L.err, (bf16*)out, lse, p.num_kv_heads,
                       p.num_chunks, p.topk, p.softmax_scale);
  };
  if (p.head_dim == 128) args(forward_kernel<128, kFwdNQ>, 256 / kFwdNQ);
  else args(forward_kernel<64, kFwdNQ>, 256 / kFwdNQ);
  return hipGetLastError();
}

}  // namespace msa
