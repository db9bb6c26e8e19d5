// Sparse forward of MSA main attention on gfx950.
//
// The pages name the flat forward (msa_bindings: sparse_atten_func) and fix
// what it must hand the backward (msa_backward_sm100: run_backward takes the
// forward's bf16 out [T, Hq, D] and fp32 lse [T, Hq]).  The kernel below is
// this library's own design for CDNA4:
//
//  * one workgroup of 4 waves per (chunk, index head): a 128-row query tile
//    of 8 tokens x 16 query heads sharing one KV head, each wave owning one
//    32-query MFMA column (2 tokens).  Workgroup ids run head-fastest, so
//    with 4 or 8 KV heads each XCD (ids are dealt to the 8 XCDs round-robin)
//    reads the K/V of one head only, which then stays in its L2;
//  * the tile's Q rows live in registers as MFMA B operands for the whole
//    chunk;
//  * per kept key block (64 keys): K and V arrive in LDS by direct
//    global->LDS loads into a K ring of three and a V ring of two swizzled
//    buffers (80 KiB at D = 128, two workgroups per CU): the copies of K of
//    block j+2 and V of block j+1 are issued while block j is consumed
//    (after its exponentials, before its O^T MFMAs), one barrier per block;
//    S^T = K Q^T (keys x queries, so a lane owns one query column), online
//    softmax in the exp2 domain with the causal mask
//    and a lazy rescale (O is rescaled only when the running max grows by
//    more than 2^8), and O^T += V^T P^T with P^T taken straight from the S^T
//    accumulators and V^T read by the LDS transpose load;
//  * out = O / l in bf16, lse = ln(sum exp(scale * s)) in fp32;
//  * P enters the O^T products as bf16.  Its rounding moves each weight by up
//    to 2^-9 relative, which shifts a row by up to about 2^-9 sum_j w_j
//    |v_j - O| before the final bf16 rounding; that matters only for rows
//    whose weight sits on a few keys, which are the rows with large |O|.  A
//    workgroup any of whose rows ends with max |O| >= 1 therefore runs its
//    tile once more in a plain loop that splits P into bf16 high and low
//    parts and multiplies both (fp32-accurate weights), and writes that
//    result instead (measured on the uniform 8K workload: about 1 % of the
//    tiles, mostly the first chunks of a document).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr float kRescaleLog2 = 8.f;
constexpr float kPreciseAbove = 1.f;  // max |O| of a row from which its tile is redone
constexpr int kFwdThreads = 256;      // 4 waves, one 32-query MFMA column each

// The next kept block of a selection row: `rem` holds the not yet taken
// slots (a wave-uniform mask), `bsel` lane s the block id of slot s.
__device__ __forceinline__ int take_block(uint64_t& rem, int bsel) {
  const int slot = (int)__builtin_ctzll(rem);
  rem &= rem - 1;
  return __builtin_amdgcn_readlane(bsel, slot);
}

// Maximum and sum over the lane pair (l, l ^ 32): one lane swap between the
// wave's halves, no LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2) void forward_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ doc_kv_off,
    const int32_t* __restrict__ sel_clean, const int32_t* __restrict__ err, bf16* __restrict__ out,
    float* __restrict__ lse, int Hkv, int C,
    int K, int sub, float scale, int T) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;           // k steps of S^T = K Q^T
  constexpr int NT = D / 32;           // 32-wide d tiles of O^T
  constexpr int NW = kFwdThreads / 64;
  constexpr int kCopyOps = kBlock / (64 / CPR) / NW;   // copies per wave for one K or V tile
  static_assert(kCopyOps < 16, "fits the low vmcnt field");
  // K ring of three, V ring of two (80 KiB at D = 128, so two workgroups
  // share a CU): K of block j+2 and V of block j+1 are copied while block j
  // is consumed.  Separate objects let the compiler see that a copy into one
  // buffer does not touch the others.
  __shared__ __attribute__((aligned(16))) bf16 kb0[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 kb1[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 kb2[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 vb0[kBlock * D];
  __shared__ __attribute__((aligned(16))) bf16 vb1[kBlock * D];

  if (err[1]) {
    fill_nan(out, (int64_t)T * Hkv * kQPerKV * D / 8, lse, (int64_t)T * Hkv * kQPerKV);
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

  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;

  // Every wave reads the selection row itself: lane s holds 64-key tile s of
  // the row (slot s with key block 64; half s % 2 of slot s / 2 with key
  // block 128), the kept tiles form a wave-uniform mask walked in order.
  const int bsel = sub_tile(sel_clean + ((int64_t)i * C + g) * K, K, sub, p0 + qcount - 1, lane);
  const uint64_t kept = __builtin_amdgcn_ballot_w64(bsel >= 0);
  const int nblk = __popcll(kept);
  uint64_t rem_k = kept, rem_v = kept, rem_c = kept;

  // Query column of this lane: tile row 32w + n32, i.e. token 2w + n32/16
  // and head n32%16.
  const int jq = 2 * w + (n32 >> 4);
  const bool qvalid = jq < qcount;
  const int pq = p0 + jq;
  const int64_t qrow = (int64_t)(tok0 + p0 + min(jq, qcount - 1)) * Hq + kQPerKV * i + (n32 & 15);
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = qvalid ? load_bf16x8(q + qrow * D + 16 * s + 8 * h) : bf16x8{};

  floatx16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = floatx16{};
  float m = -INFINITY, l = 0.f;
  const float c2 = scale * kLog2e;

  auto copy = [&](bf16* tile, const bf16* src, int b) {
    stage_block<D, NW>(tile, src, kv0, len, b, Hkv, i, w, lane);
  };
  // Issue order K0, V0, K1, then per step V_{j+1}, K_{j+2}: when block j is
  // due, only K_{j+1}'s copies may still be outstanding.
  if (nblk > 0) {
    copy(kb0, k, take_block(rem_k, bsel));
    copy(vb0, v, take_block(rem_v, bsel));
  }
  if (nblk > 1) copy(kb1, k, take_block(rem_k, bsel));

  auto consume = [&](const bf16* kt, const bf16* vt, int b, auto&& issue) {
    // S^T = K Q^T: two 32-key tiles; operands of k step s+1 are read while
    // step s runs.
    floatx16 st[2] = {floatx16{}, floatx16{}};
    // K operands three k steps ahead: fewer do not cover the LDS latency
    // (measured: two steps ahead is 2.5 % slower).
    bf16x8 ak[4][2];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      ak[s][0] = lds_row8<CPR>(kt, n32, 16 * s + 8 * h);
      ak[s][1] = lds_row8<CPR>(kt, 32 + n32, 16 * s + 8 * h);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 3 < KS) {
        ak[(s + 3) % 4][0] = lds_row8<CPR>(kt, n32, 16 * (s + 3) + 8 * h);
        ak[(s + 3) % 4][1] = lds_row8<CPR>(kt, 32 + n32, 16 * (s + 3) + 8 * h);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a) st[a] = mfma32(ak[s % 4][a], qf[s], st[a]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Online softmax.  Only the diagonal block holds keys after a query (or
    // past the document end): there, keys at block offset > klim are set to
    // -inf before the max.
    if ((b + 1) * kBlock - 1 > p0) {
      // key offset of register j of tile a: 32a + 4h + 8(j/4) + j%4
      const int klim = min(pq, len - 1) - b * kBlock - 4 * h;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          st[a][j] = 32 * a + 8 * (j >> 2) + (j & 3) <= klim ? st[a][j] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[a][j]);
    mx = max_halves(mx) * c2;   // max in the scaled log2 domain
    // Lazy rescale: the running max m only moves when a score exceeds it by
    // more than kRescaleLog2, so P = exp2(s - m) stays <= 2^kRescaleLog2 and
    // the O accumulators are rescaled only on the (rare) blocks that move it.
    const bool move = mx > m + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float m_new = move ? mx : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt] *= alpha;
      m = m_new;
    }
    const float msub = (m == -INFINITY) ? 0.f : m;
    bf16x8 pb[4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 16; ++j) pb[2 * a + (j >> 3)][j & 7] = (bf16)fast_exp2(fmaf(st[a][j], c2, -msub));
    // Row sum of the bf16 probabilities that enter O (same values normalise it).
#pragma unroll
    for (int u = 0; u < 4; ++u) l = sum_bf16x8(pb[u], l);

    // The next blocks' copies go out here, between the exponentials and the
    // O^T MFMAs (measured 2-3 % faster than right after the barrier).
    issue();
    // O^T += V^T P^T over 4 k steps of 16 keys; V^T operands double-buffered.
    bf16x8 av[2][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) av[0][tt] = lds_tr_operand_swz<CPR>(vt, 32 * tt, lane, 0, 4, 8, 12);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u + 1 < 4) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          av[(u + 1) & 1][tt] = lds_tr_operand_swz<CPR>(vt, 32 * tt, lane, 16 * (u + 1), 16 * (u + 1) + 4,
                                                        16 * (u + 1) + 8, 16 * (u + 1) + 12);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt] = mfma32(av[u & 1][tt], pb[u], o[tt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Block j: K in kb<j % 3>, V in vb<j % 2>.
  auto step = [&](int j, const bf16* kt, const bf16* vt, bf16* v_next, bf16* k_next2) {
    if (j + 1 < nblk) __builtin_amdgcn_s_waitcnt(0x0F70 | kCopyOps);   // K_{j+1} may stay in flight
    else wait_vmem();
    lds_sync();   // block j landed for every wave; all are done with block j-1's buffers
    consume(kt, vt, take_block(rem_c, bsel), [&]() {
      if (j + 1 < nblk) copy(v_next, v, take_block(rem_v, bsel));
      if (j + 2 < nblk) copy(k_next2, k, take_block(rem_k, bsel));
    });
  };
  for (int j = 0; j < nblk; j += 6) {
    step(j, kb0, vb0, vb1, kb2);
    if (j + 1 < nblk) step(j + 1, kb1, vb1, vb0, kb0);
    if (j + 2 < nblk) step(j + 2, kb2, vb0, vb1, kb1);
    if (j + 3 < nblk) step(j + 3, kb0, vb1, vb0, kb2);
    if (j + 4 < nblk) step(j + 4, kb1, vb0, vb1, kb0);
    if (j + 5 < nblk) step(j + 5, kb2, vb1, vb0, kb1);
  }

  float l_tot = sum_halves(l);
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  bool precise;
  {
    float amax = 0.f;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[tt][r]));
    const bool mine = __builtin_amdgcn_ballot_w64(qvalid && amax * inv >= kPreciseAbove) != 0;
    // One flag word per wave in a ring buffer no wave reads any more.
    int* flags = reinterpret_cast<int*>(kb2);
    lds_sync();
    if (lane == 0) flags[w] = mine;
    lds_sync();
    precise = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  }
  if (precise) {
    // The tile once more, one block at a time, with P = hi + lo.
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = floatx16{};
    m = -INFINITY;
    l = 0.f;
    uint64_t rem = kept;
    for (int j = 0; j < nblk; ++j) {
      const int b = take_block(rem, bsel);
      lds_sync();   // every wave is done with the previous block's buffers
      copy(kb0, k, b);
      copy(vb0, v, b);
      wait_vmem();
      lds_sync();
      floatx16 st[2] = {floatx16{}, floatx16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int a = 0; a < 2; ++a) st[a] = mfma32(lds_row8<CPR>(kb0, 32 * a + n32, 16 * s + 8 * h), qf[s], st[a]);
      if ((b + 1) * kBlock - 1 > p0) {
        const int klim = min(pq, len - 1) - b * kBlock - 4 * h;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj)
            st[a][jj] = 32 * a + 8 * (jj >> 2) + (jj & 3) <= klim ? st[a][jj] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, st[a][jj]);
      mx = max_halves(mx) * c2;
      if (mx > m) {
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mx);
        l *= alpha;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) o[tt] *= alpha;
        m = mx;
      }
      const float msub = (m == -INFINITY) ? 0.f : m;
      // k step u of O^T takes registers 8(u%2) .. 8(u%2)+7 of S^T tile u/2
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(fmaf(st[u >> 1][8 * (u & 1) + e], c2, -msub));
          ph[e] = (bf16)pv;
          pl[e] = (bf16)(pv - (float)ph[e]);
        }
        l = sum_bf16x8(ph, sum_bf16x8(pl, l));
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const bf16x8 av = lds_tr_operand_swz<CPR>(vb0, 32 * tt, lane, 16 * u, 16 * u + 4, 16 * u + 8,
                                                    16 * u + 12);
          o[tt] = mfma32(av, ph, o[tt]);
          o[tt] = mfma32(av, pl, o[tt]);
        }
      }
    }
    l_tot = sum_halves(l);
    inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  }

  if (!qvalid) return;
  bf16* orow = out + qrow * D;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = (bf16)(o[tt][4 * jg + r] * inv);
      store_bf16x4(orow + 32 * tt + 8 * jg + 4 * h, v4);
    }
  }
  if (h == 0) lse[qrow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
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
                       sched + L.doc_kv_off, sched + L.sel_clean, sched + L.err, (bf16*)out, lse,
                       p.num_kv_heads,
                       p.num_chunks, p.topk, p.block_size / kBlock, p.softmax_scale, p.total_tokens);
  };
  if (p.head_dim == 128) args(forward_kernel<128>, kFwdThreads);
  else args(forward_kernel<64>, kFwdThreads);
  return hipGetLastError();
}

}  // namespace msa
