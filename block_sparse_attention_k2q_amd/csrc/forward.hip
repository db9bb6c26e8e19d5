// Sparse forward of MSA main attention on gfx950.
//
// The pages name the flat forward (msa_bindings: sparse_atten_func) and fix
// what it must hand the backward (msa_backward_sm100: run_backward takes the
// forward's bf16 out [T, Hq, D] and fp32 lse [T, Hq]).  The kernel below is
// this library's own design for CDNA4:
//
//  * one workgroup per (chunk, index head): a 128-row query tile of 8 tokens
//    x 16 query heads that share one KV head; workgroup ids run head-fastest
//    so that, with 4 or 8 KV heads, each XCD (ids are dealt to the 8 XCDs
//    round-robin) only ever reads the K/V of one head;
//  * 4 waves, each owning 32 query rows (2 tokens x 16 heads); the tile's Q
//    rows live in registers as MFMA B operands for the whole chunk;
//  * per kept key block (64 keys): K and V are staged in LDS (next block
//    prefetched into registers while the current one is consumed),
//    S^T = K Q^T (keys x queries) so that every lane owns one query column,
//    online softmax in the exp2 domain with the causal mask on the diagonal
//    block, and O^T += V^T P^T with P^T taken straight from the S^T
//    accumulators (V^T read with the LDS transpose load);
//  * out = O / l in bf16, lse = ln(sum exp(scale * s)) in fp32.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kFwdThreads = 256;

template <int D>
struct FwdSmem {
  static constexpr int LDK = D + 8;    // padded row pitch of the K tile (bf16 elements)
  static constexpr int LDV = D + 16;   // padded row pitch of the V tile
  bf16 k[kBlock * LDK];
  bf16 v[kBlock * LDV];
  int blocks[64];
  int nblocks;
};

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2) void forward_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
    const int32_t* __restrict__ doc_chunk_off, const int32_t* __restrict__ sel_clean,
    const int32_t* __restrict__ err, bf16* __restrict__ out, float* __restrict__ lse, int Hkv, int C,
    int K, float scale) {
  using S = FwdSmem<D>;
  constexpr int LDK = S::LDK, LDV = S::LDV;
  constexpr int KS = D / 16;           // k steps of S^T = K Q^T
  constexpr int NT = D / 32;           // 32-wide d tiles of O^T
  constexpr int VEC = D / 8;           // 16-byte vectors per K/V row
  constexpr int PF = kBlock * VEC / kFwdThreads;  // prefetch vectors per thread per tensor
  __shared__ __attribute__((aligned(16))) S sm;

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

  if (threadIdx.x == 0) {
    int n = 0;
    const int32_t* row = sel_clean + ((int64_t)i * C + g) * K;
    for (int s = 0; s < K; ++s) {
      const int b = row[s];
      if (b >= 0) sm.blocks[n++] = b;
    }
    sm.nblocks = n;
  }

  const int w = wave_id(), lane = lane_id();
  const int n32 = lane & 31, h = lane >> 5;
  const int jq = 2 * w + (n32 >> 4);         // token of this lane's query column
  const int hh = n32 & 15;
  const bool qvalid = jq < qcount;
  const int pq = p0 + jq;                    // document-local query position
  const int64_t qrow = (int64_t)(tok0 + p0 + jq) * Hq + kQPerKV * i + hh;

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qvalid) qf[s] = load_bf16x8(q + qrow * D + 16 * s + 8 * h);
    else qf[s] = bf16x8{};
  }

  floatx16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = floatx16{};
  float m = -INFINITY, l = 0.f;
  const float c2 = scale * kLog2e;

  lds_barrier();
  const int nblk = sm.nblocks;

  // Register prefetch of one block's K and V rows (zero past the document end).
  u32x4 pk[PF], pv[PF];
  auto prefetch = [&](int b) {
#pragma unroll
    for (int x = 0; x < PF; ++x) {
      const int e = threadIdx.x + x * kFwdThreads;
      const int row = e / VEC, col = (e % VEC) * 8;
      const int key = b * kBlock + row;
      if (key < len) {
        const int64_t off = ((int64_t)(tok0 + key) * Hkv + i) * D + col;
        pk[x] = *reinterpret_cast<const u32x4*>(k + off);
        pv[x] = *reinterpret_cast<const u32x4*>(v + off);
      } else {
        pk[x] = u32x4{0, 0, 0, 0};
        pv[x] = u32x4{0, 0, 0, 0};
      }
    }
  };
  if (nblk > 0) prefetch(sm.blocks[0]);

  for (int bi = 0; bi < nblk; ++bi) {
    const int b = sm.blocks[bi];
    lds_barrier();  // all waves are done with the previous block's tiles
#pragma unroll
    for (int x = 0; x < PF; ++x) {
      const int e = threadIdx.x + x * kFwdThreads;
      const int row = e / VEC, col = (e % VEC) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[row * LDK + col]) = pk[x];
      *reinterpret_cast<u32x4*>(&sm.v[row * LDV + col]) = pv[x];
    }
    lds_barrier();
    if (bi + 1 < nblk) prefetch(sm.blocks[bi + 1]);

    // S^T = K Q^T: two 32-key tiles.
    floatx16 st[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = load_bf16x8(&sm.k[(32 * t + n32) * LDK + 16 * s + 8 * h]);
        st[t] = mfma32(a, qf[s], st[t]);
      }
    }

    // Scores in the log2 domain; causal mask only where the block can hold
    // keys after this query (the diagonal block).
    const bool need_mask = (b + 1) * kBlock - 1 > p0;
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = st[t][j] * c2;
        if (need_mask) {
          const int key = b * kBlock + 32 * t + 8 * (j >> 2) + 4 * h + (j & 3);
          if (key > pq || key >= len) x = -INFINITY;
        }
        st[t][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv_ = fast_exp2(st[t][j] - msub);
        psum += pv_;
        pb[2 * t + (j >> 3)][j & 7] = (bf16)pv_;
      }
    }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] *= alpha;

    // O^T += V^T P^T over the 4 k steps of 16 keys.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 a = lds_tr_operand(sm.v, LDV, 32 * t, lane, 16 * u, 16 * u + 4, 16 * u + 8,
                                        16 * u + 12);
        o[t] = mfma32(a, pb[u], o[t]);
      }
    }
  }

  const float l_tot = l + swap_halves(l);
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  bf16* orow = out + qrow * D;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = (bf16)(o[t][4 * jg + r] * inv);
      store_bf16x4(orow + 32 * t + 8 * jg + 4 * h, v4);
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
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kFwdThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, cu, sched + L.chunk_doc, sched + L.doc_chunk_off,
                       sched + L.sel_clean, sched + L.err, (bf16*)out, lse, p.num_kv_heads,
                       p.num_chunks, p.topk, p.softmax_scale);
  };
  if (p.head_dim == 128) args(forward_kernel<128>);
  else args(forward_kernel<64>);
  return hipGetLastError();
}

}  // namespace msa
