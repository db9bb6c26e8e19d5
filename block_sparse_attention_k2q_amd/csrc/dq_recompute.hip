// dQ kernel of the MSA_DQ_RECOMPUTE mode of the backward on gfx950 (the
// default mode's dq_from_ds_kernel is in dq.hip; the two are separate files
// because they compile best with different instruction-scheduling flags).
//
// dQ_p = scale * sum_j dS_pj k_j with dS = P (dP - Delta), P = exp(s - LSE)
// (msa_backward_sm100 page: the dQ^T contraction; kernels page: Delta from
// the backward preprocess).  On MI355X, fp32 global atomics execute beyond
// the L2 at a rate that cannot keep up with one 128 x D atomic tile per
// (chunk, block) pair, so instead of scattering dQ from the KV-parallel
// kernel this kernel walks each chunk's kept blocks, like the forward, and
// keeps dQ in registers:
//
//  * one workgroup per (chunk, index head), 4 waves x 32 query rows; Q and
//    dO rows of the tile stay in registers as MFMA B operands;
//  * per kept 64-key tile (a selected block of 128 keys is two tiles; a tile
//    whose first key lies after the chunk's last query is dropped): K and V
//    arrive in one of two swizzled LDS buffers by
//    direct global->LDS loads (next block in flight while the current one is
//    consumed), S^T = K Q^T and dP^T = V dO^T (keys x queries),
//    P^T = exp2(S^T * scale * log2e - LSE * log2e) with the causal mask,
//    dS^T = P^T (dP^T - Delta), and dQ^T += K^T dS^T with dS^T taken straight
//    from the accumulators and K^T read through the LDS transpose load;
//  * dq = bf16(scale * dQ) written once.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kDqThreads = 256;

template <int D>
__global__ __launch_bounds__(kDqThreads, 2) void dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ doc_kv_off,
    const int32_t* __restrict__ sel_clean, const int32_t* __restrict__ err, bf16* __restrict__ dq, int Hkv,
    int C, int K, int sub, float scale, int T) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;
  constexpr int NT = D / 32;
  constexpr int NW = kDqThreads / 64;
  __shared__ __attribute__((aligned(16))) KVTiles<D> buf0;
  __shared__ __attribute__((aligned(16))) KVTiles<D> buf1;
  __shared__ int s_blocks[64];   // kept 64-key tiles (a block of 128 keys is two)
  __shared__ int s_slots[64];
  __shared__ int s_nblocks;

  if (err[1]) {
    fill_nan(dq, (int64_t)T * Hkv * kQPerKV * D / 8, nullptr, 0);
    return;
  }
  const int i = blockIdx.x % Hkv;
  const int g = blockIdx.x / Hkv;
  const int d = chunk_doc[g];
  const int c = g - doc_chunk_off[d];
  const int tok0 = cu[d];
  const int len = cu[d + 1] - tok0;
  const int kv0 = doc_kv_off[d];       // the document's first row of k and v
  const int p0 = kChunk * c;
  const int qcount = min(kChunk, len - p0);
  const int Hq = Hkv * kQPerKV;

  if (threadIdx.x < 64) {
    const int n = compact_tiles(sel_clean + ((int64_t)i * C + g) * K, K, sub, p0 + qcount - 1, threadIdx.x,
                                s_blocks, s_slots);
    if (threadIdx.x == 0) s_nblocks = n;
  }

  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;
  const int jq = 2 * w + (n32 >> 4);
  const int hh = n32 & 15;
  const bool qvalid = jq < qcount;
  const int pq = p0 + jq;
  const int64_t qrow = (int64_t)(tok0 + p0 + min(jq, qcount - 1)) * Hq + kQPerKV * i + hh;

  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qvalid ? load_bf16x8(q + qrow * D + 16 * s + 8 * h) : bf16x8{};
    of[s] = qvalid ? load_bf16x8(dout + qrow * D + 16 * s + 8 * h) : bf16x8{};
  }
  const float lv = lse[qrow];
  const float l2 = (qvalid && lv != -INFINITY) ? lv * kLog2e : INFINITY;
  const float dl = qvalid ? delta[qrow] : 0.f;
  const float c2 = scale * kLog2e;

  floatx16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx16{};

  lds_barrier();
  const int nblk = s_nblocks;
  if (nblk > 0) stage_kv<D, NW>(buf0, k, v, kv0, len, s_blocks[0], Hkv, i, w, lane);

  auto consume = [&](const KVTiles<D>& t, int b) {
    // S^T = K Q^T and dP^T = V dO^T, operands of step s+1 read during step s.
    floatx16 st[2] = {floatx16{}, floatx16{}};
    floatx16 dpt[2] = {floatx16{}, floatx16{}};
    bf16x8 ak[2][2], av[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      ak[0][a] = lds_row8<CPR>(t.k, 32 * a + n32, 8 * h);
      av[0][a] = lds_row8<CPR>(t.v, 32 * a + n32, 8 * h);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          ak[(s + 1) & 1][a] = lds_row8<CPR>(t.k, 32 * a + n32, 16 * (s + 1) + 8 * h);
          av[(s + 1) & 1][a] = lds_row8<CPR>(t.v, 32 * a + n32, 16 * (s + 1) + 8 * h);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        st[a] = mfma32(ak[s & 1][a], qf[s], st[a]);
        dpt[a] = mfma32(av[s & 1][a], of[s], dpt[a]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // dS^T in bf16, packed as B operands of dQ^T (k step u = keys 16u..16u+15).
    // Only the diagonal block holds keys after a query (or past the document
    // end); there those scores become -inf, so P = 0.
    if ((b + 1) * kBlock - 1 > p0) {
      const int klim = min(pq, len - 1) - b * kBlock;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = 32 * a + 8 * (j >> 2) + 4 * h + (j & 3);
          st[a][j] = key <= klim ? st[a][j] : -INFINITY;
        }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = fast_exp2(fmaf(st[a][j], c2, -l2));
        dsb[2 * a + (j >> 3)][j & 7] = (bf16)(pv * (dpt[a][j] - dl));
      }

    // dQ^T += K^T dS^T, K^T operands double-buffered.
    bf16x8 kt[2][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) kt[0][tt] = lds_tr_operand_swz<CPR>(t.k, 32 * tt, lane, 0, 4, 8, 12);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u + 1 < 4) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          kt[(u + 1) & 1][tt] = lds_tr_operand_swz<CPR>(t.k, 32 * tt, lane, 16 * (u + 1), 16 * (u + 1) + 4,
                                                        16 * (u + 1) + 8, 16 * (u + 1) + 12);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma32(kt[u & 1][tt], dsb[u], acc[tt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int bi = 0; bi < nblk; bi += 2) {
    // Even blocks use buf0, odd blocks buf1.
    wait_vmem();
    lds_barrier();   // block bi landed in buf0; all waves are done with buf1
    if (bi + 1 < nblk) stage_kv<D, NW>(buf1, k, v, kv0, len, s_blocks[bi + 1], Hkv, i, w, lane);
    consume(buf0, s_blocks[bi]);
    if (bi + 1 < nblk) {
      wait_vmem();
      lds_barrier();  // block bi+1 landed in buf1; all waves are done with buf0
      if (bi + 2 < nblk) stage_kv<D, NW>(buf0, k, v, kv0, len, s_blocks[bi + 2], Hkv, i, w, lane);
      consume(buf1, s_blocks[bi + 1]);
    }
  }

  if (!qvalid) return;
  bf16* orow = dq + qrow * D;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = (bf16)(acc[t][4 * jg + r] * scale);
      store_bf16x4(orow + 32 * t + 8 * jg + 4 * h, v4);
    }
  }
}

}  // namespace

hipError_t launch_dq_recompute(const msa_problem& p, const void* q, const void* k, const void* v,
                               const void* dout, const float* lse, const int32_t* cu, const int32_t* sched,
                               const msa_schedule_layout& L, const void* scratch, void* dq,
                               hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_chunks * p.num_kv_heads;
  if (nwg == 0) return hipSuccess;
  const BackwardScratch S = backward_scratch_layout(p);
  const float* delta = (const float*)((const uint8_t*)scratch + S.delta);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kDqThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, delta, cu,
                       sched + L.chunk_doc, sched + L.doc_chunk_off, sched + L.doc_kv_off, sched + L.sel_clean,
                       sched + L.err, (bf16*)dq, p.num_kv_heads, p.num_chunks, p.topk, p.block_size / kBlock,
                       p.softmax_scale, p.total_tokens);
  };
  if (p.head_dim == 128) go(dq_kernel<128>);
  else go(dq_kernel<64>);
  return hipGetLastError();
}

}  // namespace msa
