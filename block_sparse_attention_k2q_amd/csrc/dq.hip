// dQ from the stored dS (MSA_DQ_DS_BUFFER, the default mode of the MSA
// backward) on gfx950; the MSA_DQ_RECOMPUTE mode's kernel is in
// dq_recompute.hip.  Both walk a chunk's kept 64-key tiles (a selected block
// of 128 keys is two tiles).
//
// dQ_p = scale * sum_j dS_pj k_j (msa_backward_sm100 page: the dQ^T
// contraction).  On MI355X, fp32 global atomics execute beyond the L2 at a
// rate that cannot keep up with one 128 x D atomic tile per (chunk, block)
// pair, so instead of scattering dQ from the KV-parallel kernel, that kernel
// stores each tile's bf16 dS and this kernel walks each chunk's kept
// blocks, like the forward, keeping dQ in registers.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kDqThreads = 256;

// dQ from stored dS (MSA_DQ_DS_BUFFER): one workgroup per (chunk, index
// head), 4 waves x 32 query rows.  The chunk's kept 64-key tiles ("blocks"
// below) stream through a three-stage ring: while block n is consumed, blocks n+1 and n+2 are in
// flight (K by direct loads into one of three swizzled LDS buffers, the
// wave's dS^T operands, stored by the main kernel in MFMA operand order so
// that each 16-key step is one contiguous 1 KiB load per wave, into
// registers).  dQ^T += K^T dS^T per block;
// dq = bf16(scale * dQ) written once.
template <int D>
__global__ __launch_bounds__(kDqThreads, 2) void dq_from_ds_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ ds, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_doc, const int32_t* __restrict__ doc_chunk_off,
    const int32_t* __restrict__ doc_kv_off, const int32_t* __restrict__ sel_clean,
    const int32_t* __restrict__ err, bf16* __restrict__ dq,
    int Hkv, int C, int K, int sub, float scale, int T) {
  constexpr int CPR = D / 8;
  constexpr int NT = D / 32;
  constexpr int NW = kDqThreads / 64;
  // vector-memory operations one block costs a wave: K copies + 4 dS loads
  constexpr int kOpsPerBlock = kBlock / (64 / CPR) / NW + 4;
  static_assert(kOpsPerBlock < 16, "fits the low vmcnt field");
  __shared__ __attribute__((aligned(16))) bf16 kbuf0[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 kbuf1[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 kbuf2[kBlock * D];
  __shared__ int s_slot[64];
  __shared__ int s_block[64];
  __shared__ int s_n;

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
  const int kv0 = doc_kv_off[d];       // the document's first row of k
  const int p0 = kChunk * c;
  const int qcount = min(kChunk, len - p0);
  const int Hq = Hkv * kQPerKV;
  const int64_t row_base = ((int64_t)i * C + g) * K;

  if (threadIdx.x < 64) {
    const int n = compact_tiles(sel_clean + row_base, K, sub, p0 + qcount - 1, threadIdx.x, s_block, s_slot);
    if (threadIdx.x == 0) s_n = n;
  }

  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;
  const int jq = 2 * w + (n32 >> 4);
  const bool qvalid = jq < qcount;
  const int64_t qrow = (int64_t)(tok0 + p0 + min(jq, qcount - 1)) * Hq + kQPerKV * i + (n32 & 15);
  // this lane's dS^T operand of step u: 8 bf16 at ((4w + u) * 64 + lane) * 8 in a slot
  const bf16* ds_lane = ds + row_base * sub * (kDsSlotBytes / 2) + w * 4 * 512 + lane * 8;

  floatx16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx16{};

  lds_barrier();
  const int nblk = s_n;
  bf16x8 d0[4], d1[4], d2[4];
  auto issue = [&](int n, bf16* kb, bf16x8 (&dst)[4]) {
    stage_block<D, NW>(kb, k, kv0, len, s_block[n], Hkv, i, w, lane);
    const bf16* src = ds_lane + (int64_t)s_slot[n] * (kDsSlotBytes / 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = load_bf16x8_stream(src + 512 * u);
  };
  auto step = [&](int n, const bf16* kb, const bf16x8 (&dc)[4], bf16* next_kb, bf16x8 (&next_d)[4]) {
    // Block n's copies are done once at most the next block's are pending.
    if (n + 1 < nblk) __builtin_amdgcn_s_waitcnt(0x0F70 | kOpsPerBlock);
    else wait_vmem();
    // LDS-only barrier: a release fence would also wait for block n + 1
    lds_sync();      // block n landed for every wave; all are done with block n - 1
    if (n + 2 < nblk) issue(n + 2, next_kb, next_d);
    bf16x8 kt[2][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) kt[0][tt] = lds_tr_operand_swz<CPR>(kb, 32 * tt, lane, 0, 4, 8, 12);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u + 1 < 4) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          kt[(u + 1) & 1][tt] = lds_tr_operand_swz<CPR>(kb, 32 * tt, lane, 16 * (u + 1), 16 * (u + 1) + 4,
                                                        16 * (u + 1) + 8, 16 * (u + 1) + 12);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma32(kt[u & 1][tt], dc[u], acc[tt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nblk > 0) issue(0, kbuf0, d0);
  if (nblk > 1) issue(1, kbuf1, d1);
  for (int bi = 0; bi < nblk; bi += 3) {
    // block bi + j uses kbuf<j> and d<j>; the block issued at step n takes
    // the buffers of block n - 1
    step(bi, kbuf0, d0, kbuf2, d2);
    if (bi + 1 < nblk) step(bi + 1, kbuf1, d1, kbuf0, d0);
    if (bi + 2 < nblk) step(bi + 2, kbuf2, d2, kbuf1, d1);
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

hipError_t launch_backward_dq(const msa_problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const int32_t* cu,
                              const int32_t* sched, const msa_schedule_layout& L, const void* scratch,
                              void* dq, hipStream_t stream) {
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL || p.dq_mode == MSA_DQ_ATOMIC_POOL_BF16) return hipSuccess;
  const int64_t nwg = (int64_t)p.num_chunks * p.num_kv_heads;
  if (nwg == 0) return hipSuccess;
  const BackwardScratch S = backward_scratch_layout(p);
  if (p.dq_mode == MSA_DQ_DS_BUFFER) {
    auto go_ds = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kDqThreads), 0, stream, (const bf16*)k,
                         (const bf16*)((const uint8_t*)scratch + S.ds), cu, sched + L.chunk_doc,
                         sched + L.doc_chunk_off, sched + L.doc_kv_off, sched + L.sel_clean, sched + L.err,
                         (bf16*)dq, p.num_kv_heads, p.num_chunks, p.topk, p.block_size / kBlock,
                         p.softmax_scale, p.total_tokens);
    };
    if (p.head_dim == 128) go_ds(dq_from_ds_kernel<128>);
    else go_ds(dq_from_ds_kernel<64>);
    return hipGetLastError();
  }
  return launch_dq_recompute(p, q, k, v, dout, lse, cu, sched, L, scratch, dq, stream);
}

}  // namespace msa
