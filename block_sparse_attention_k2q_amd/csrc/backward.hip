// KV-parallel backward of MSA main attention on gfx950.
//
// Pages: msa_backward_sm100 (module description: each CTA walks task rows of
// 8 queries x 16 heads = one 128-row tile, bucketed by (index head, key
// block); K/V resident per bucket, Q/dO loaded per tile; five GEMMs S^T,
// dP^T, dV, dK, dQ; dV/dK accumulated per bucket segment and flushed with
// fp32 atomics; dQ scattered per tile; run_backward returns bf16 dq/dk/dv),
// kernels page (preprocess / postprocess submodules), msa_schedule (walk
// rule).  The dQ pool is fp32 here.
//
// Main kernel design on CDNA4 (4 waves, one workgroup walks [lo, hi) of the
// task table):
//  * on a bucket change: flush the dK/dV accumulators of the previous bucket
//    segment with fp32 atomics, then stage the new block's K and V in LDS;
//  * per task row: stage the 128 Q and dO rows (8 tokens x 16 heads) in LDS,
//    with LSE * log2(e) and Delta for each row;
//  * wave w owns query rows 32w..32w+31 for S^T = K Q^T and dP^T = V dO^T
//    (keys x queries, so each lane owns one query column), computes
//    P^T = exp2(S^T * scale * log2e - LSE * log2e) (causal mask on the
//    diagonal block) and dS^T = P^T (dP^T - Delta);
//  * dQ = dS K runs straight from the dS^T accumulators (its contraction is
//    over keys, the accumulator row index) with K read through the LDS
//    transpose load, then goes to the fp32 pool with atomics: 32 lanes add
//    32 consecutive floats of one row;
//  * P^T and dS^T go to LDS as bf16; wave w then owns a slice of the dV and
//    dK outputs (keys x d) and contracts over all 128 query rows, reading P,
//    dS, dO and Q through the transpose load.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// Preprocess: Delta = rowsum(dO * O) in fp32; zero the dQ pool and dK/dV.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const bf16* __restrict__ out,
                                                         const bf16* __restrict__ dout,
                                                         float* __restrict__ delta,
                                                         float* __restrict__ dq_pool,
                                                         float* __restrict__ dkv, int64_t n_vec,
                                                         int64_t n_dkv_vec) {
  constexpr int LPR = D / 8;  // lanes per (token, head) row
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x < n_dkv_vec) {
    floatx4* p = reinterpret_cast<floatx4*>(dkv) + 2 * x;
    p[0] = floatx4{};
    p[1] = floatx4{};
  }
  if (x >= n_vec) return;  // n_vec is a multiple of LPR, so row groups stay whole
  const bf16x8 a = load_bf16x8(out + 8 * x);
  const bf16x8 b = load_bf16x8(dout + 8 * x);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)b[e];
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off, 64);
  if ((x % LPR) == 0) delta[x / LPR] = s;
  floatx4* p = reinterpret_cast<floatx4*>(dq_pool) + 2 * x;
  p[0] = floatx4{};
  p[1] = floatx4{};
}

// ---------------------------------------------------------------------------
// Postprocess: dq = bf16(scale * pool), dk = bf16(scale * dk_acc), dv = bf16(dv_acc).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void postprocess_kernel(const float* __restrict__ dq_pool,
                                                          const float* __restrict__ dk_acc,
                                                          const float* __restrict__ dv_acc,
                                                          bf16* __restrict__ dq, bf16* __restrict__ dk,
                                                          bf16* __restrict__ dv, int64_t n_q_vec,
                                                          int64_t n_kv_vec, float scale) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  auto cast8 = [](const float* src, bf16* dst, float mul) {
    const floatx4 a = reinterpret_cast<const floatx4*>(src)[0];
    const floatx4 b = reinterpret_cast<const floatx4*>(src)[1];
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (bf16)(a[e] * mul);
      r[4 + e] = (bf16)(b[e] * mul);
    }
    store_bf16x8(dst, r);
  };
  if (x < n_q_vec) cast8(dq_pool + 8 * x, dq + 8 * x, scale);
  if (x < n_kv_vec) {
    cast8(dk_acc + 8 * x, dk + 8 * x, scale);
    cast8(dv_acc + 8 * x, dv + 8 * x, 1.f);
  }
}

// ---------------------------------------------------------------------------
// Main kernel.
// ---------------------------------------------------------------------------
template <int D>
struct BwdSmem {
  static constexpr int LDK = D + 8;      // K, V, Q, dO row pitch (bf16 elements)
  static constexpr int LDP = kBlock + 8; // P, dS row pitch
  bf16 k[kBlock * LDK];
  bf16 v[kBlock * LDK];
  bf16 q[kTileM * LDK];
  bf16 dout[kTileM * LDK];
  bf16 p[kTileM * LDP];
  bf16 ds[kTileM * LDP];
  float lse2[kTileM];
  float delta[kTileM];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void backward_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ task_meta,
    const int32_t* __restrict__ desc, const int32_t* __restrict__ err, float* __restrict__ dq_pool,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, int Hkv, float scale) {
  using S = BwdSmem<D>;
  constexpr int LDK = S::LDK, LDP = S::LDP;
  constexpr int KS = D / 16;                 // k steps over d
  constexpr int NT = D / 32;                 // 32-wide d tiles
  constexpr int VEC = D / 8;                 // 16-byte vectors per row
  constexpr int OUT_TILES = 2 * NT / 4;      // dV (and dK) output tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  if (err[1]) return;
  const int grid_walks = desc[5];
  const int wg = blockIdx.x;
  if (wg >= grid_walks) return;
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

  // Output tiles of dV/dK owned by this wave: (key tile mt, d tile nt).
  int own_mt[OUT_TILES], own_nt[OUT_TILES];
#pragma unroll
  for (int x = 0; x < OUT_TILES; ++x) {
    const int tile = w * OUT_TILES + x;  // tiles numbered d-tile major
    own_nt[x] = tile / 2;
    own_mt[x] = tile % 2;
  }
  floatx16 acc_dv[OUT_TILES], acc_dk[OUT_TILES];

  int cur_i = -1, cur_r = -1, cur_tok0 = 0, cur_len = 0, cur_b = 0;

  auto flush = [&]() {
#pragma unroll
    for (int x = 0; x < OUT_TILES; ++x) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 32 * own_mt[x] + 8 * (j >> 2) + 4 * h + (j & 3);
        const int kpos = cur_b * kBlock + key;
        if (kpos < cur_len) {
          const int64_t off = ((int64_t)(cur_tok0 + kpos) * Hkv + cur_i) * D + 32 * own_nt[x] + n32;
          atomicAdd(dv_acc + off, acc_dv[x][j]);
          atomicAdd(dk_acc + off, acc_dk[x][j]);
        }
      }
    }
  };

  for (int row = lo; row < hi; ++row) {
    const int32_t* tm = task_meta + (int64_t)row * 6;
    const int i = tm[0], r = tm[1], qb = tm[2], qc = tm[3], d = tm[4], b = tm[5];
    const int tok0 = cu[d];
    const int len = cu[d + 1] - tok0;
    __syncthreads();  // previous tile fully consumed
    if (i != cur_i || r != cur_r) {
      if (cur_i >= 0) flush();
#pragma unroll
      for (int x = 0; x < OUT_TILES; ++x) {
        acc_dv[x] = floatx16{};
        acc_dk[x] = floatx16{};
      }
      cur_i = i; cur_r = r; cur_tok0 = tok0; cur_len = len; cur_b = b;
      for (int e = threadIdx.x; e < kBlock * VEC; e += kBwdThreads) {
        const int kr = e / VEC, col = (e % VEC) * 8;
        const int kpos = b * kBlock + kr;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (kpos < len) {
          const int64_t off = ((int64_t)(tok0 + kpos) * Hkv + i) * D + col;
          kv = *reinterpret_cast<const u32x4*>(k + off);
          vv = *reinterpret_cast<const u32x4*>(v + off);
        }
        *reinterpret_cast<u32x4*>(&sm.k[kr * LDK + col]) = kv;
        *reinterpret_cast<u32x4*>(&sm.v[kr * LDK + col]) = vv;
      }
    }
    // Q / dO tile rows m = token * 16 + head; rows past the document end are zero.
    for (int e = threadIdx.x; e < kTileM * VEC; e += kBwdThreads) {
      const int m = e / VEC, col = (e % VEC) * 8;
      const int j = m >> 4, hh = m & 15;
      u32x4 qv = {0, 0, 0, 0}, ov = {0, 0, 0, 0};
      if (j < qc) {
        const int64_t off = ((int64_t)(tok0 + qb + j) * Hq + kQPerKV * i + hh) * D + col;
        qv = *reinterpret_cast<const u32x4*>(q + off);
        ov = *reinterpret_cast<const u32x4*>(dout + off);
      }
      *reinterpret_cast<u32x4*>(&sm.q[m * LDK + col]) = qv;
      *reinterpret_cast<u32x4*>(&sm.dout[m * LDK + col]) = ov;
    }
    if (threadIdx.x < kTileM) {
      const int m = threadIdx.x, j = m >> 4, hh = m & 15;
      float l2 = INFINITY, dl = 0.f;
      if (j < qc) {
        const int64_t rowi = (int64_t)(tok0 + qb + j) * Hq + kQPerKV * i + hh;
        const float lv = lse[rowi];
        l2 = (lv == -INFINITY) ? INFINITY : lv * kLog2e;
        dl = delta[rowi];
      }
      sm.lse2[m] = l2;
      sm.delta[m] = dl;
    }
    __syncthreads();

    // --- S^T and dP^T for this wave's 32 query rows -------------------------
    const int mq = 32 * w + n32;   // this lane's query row in the tile
    floatx16 st[2] = {floatx16{}, floatx16{}};
    floatx16 dpt[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 bq = load_bf16x8(&sm.q[mq * LDK + 16 * s + 8 * h]);
      const bf16x8 bo = load_bf16x8(&sm.dout[mq * LDK + 16 * s + 8 * h]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 ak = load_bf16x8(&sm.k[(32 * t + n32) * LDK + 16 * s + 8 * h]);
        const bf16x8 av = load_bf16x8(&sm.v[(32 * t + n32) * LDK + 16 * s + 8 * h]);
        st[t] = mfma32(ak, bq, st[t]);
        dpt[t] = mfma32(av, bo, dpt[t]);
      }
    }
    const float l2 = sm.lse2[mq];
    const float dl = sm.delta[mq];
    const int pq = qb + (mq >> 4);
    const bool need_mask = (b + 1) * kBlock - 1 > qb;
    bf16x8 dsa[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4 p4, d4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int j = 4 * jg + rr;
          float pv = fast_exp2(st[t][j] * c2 - l2);
          if (need_mask) {
            const int kpos = b * kBlock + 32 * t + 8 * jg + 4 * h + rr;
            if (kpos > pq || kpos >= len) pv = 0.f;
          }
          const float dsv = pv * (dpt[t][j] - dl);
          p4[rr] = (bf16)pv;
          d4[rr] = (bf16)dsv;
          dsa[2 * t + (jg >> 1)][4 * (jg & 1) + rr] = d4[rr];
        }
        // P and dS rows of this query, keys 32t + 8jg + 4h .. +3
        store_bf16x4(&sm.p[mq * LDP + 32 * t + 8 * jg + 4 * h], p4);
        store_bf16x4(&sm.ds[mq * LDP + 32 * t + 8 * jg + 4 * h], d4);
      }
    }

    // --- dQ = dS K (32 query rows x D) -> fp32 pool ---------------------------
    {
      floatx16 dq[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) dq[t] = floatx16{};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 bk = lds_tr_operand(sm.k, LDK, 32 * t, lane, 16 * u, 16 * u + 4, 16 * u + 8,
                                           16 * u + 12);
          dq[t] = mfma32(dsa[u], bk, dq[t]);
        }
      }
      // accumulator: column = d (lane), rows = query rows 8(j/4) + 4h + j%4 of this wave
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
        const int jt = m >> 4, hh = m & 15;
        if (jt < qc) {
          float* dst = dq_pool + ((int64_t)(tok0 + qb + jt) * Hq + kQPerKV * i + hh) * D + n32;
#pragma unroll
          for (int t = 0; t < NT; ++t) atomicAdd(dst + 32 * t, dq[t][j]);
        }
      }
    }
    __syncthreads();  // P, dS complete in LDS

    // --- dV += P^T dO, dK += dS^T Q over all 128 query rows -------------------
#pragma unroll
    for (int u = 0; u < kTileM / 16; ++u) {
#pragma unroll
      for (int x = 0; x < OUT_TILES; ++x) {
        const int mt = own_mt[x], nt = own_nt[x];
        const bf16x8 ap = lds_tr_operand(sm.p, LDP, 32 * mt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                         16 * u + 12);
        const bf16x8 bo = lds_tr_operand(sm.dout, LDK, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                         16 * u + 12);
        acc_dv[x] = mfma32(ap, bo, acc_dv[x]);
        const bf16x8 ad = lds_tr_operand(sm.ds, LDP, 32 * mt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                         16 * u + 12);
        const bf16x8 bq = lds_tr_operand(sm.q, LDK, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                         16 * u + 12);
        acc_dk[x] = mfma32(ad, bq, acc_dk[x]);
      }
    }
  }
  if (cur_i >= 0) flush();
}

}  // namespace

hipError_t launch_backward_preprocess(const msa_problem& p, const void* out, const void* dout,
                                      void* scratch, hipStream_t stream) {
  const BackwardScratch L = backward_scratch_layout(p);
  uint8_t* base = (uint8_t*)scratch;
  const int64_t hq = (int64_t)p.num_kv_heads * p.q_per_kv;
  const int64_t n_vec = (int64_t)p.total_tokens * hq * p.head_dim / 8;
  // dK and dV accumulators are adjacent: zero both as one range.
  const int64_t n_dkv_vec = (int64_t)(L.total - L.dk_acc) / 32;
  const int64_t n = n_vec > n_dkv_vec ? n_vec : n_dkv_vec;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, (const bf16*)out, (const bf16*)dout,
                       (float*)(base + L.delta), (float*)(base + L.dq_pool), (float*)(base + L.dk_acc),
                       n_vec, n_dkv_vec);
  };
  if (p.head_dim == 128) go(preprocess_kernel<128>);
  else go(preprocess_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_backward_main(const msa_problem& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const int32_t* cu,
                                const int32_t* sched, const msa_schedule_layout& L, void* scratch,
                                hipStream_t stream) {
  const BackwardScratch S = backward_scratch_layout(p);
  uint8_t* base = (uint8_t*)scratch;
  const int64_t cap = (int64_t)p.num_kv_heads * p.num_chunks * p.topk;
  const int64_t grid = grid_launch_bound(cap, p.num_cus);
  auto go = [&](auto kern, size_t lds) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBwdThreads), lds, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                       (const float*)(base + S.delta), cu, sched + L.task_meta, sched + L.desc,
                       sched + L.err, (float*)(base + S.dq_pool), (float*)(base + S.dk_acc),
                       (float*)(base + S.dv_acc), p.num_kv_heads, p.softmax_scale);
    return hipGetLastError();
  };
  if (p.head_dim == 128) return go(backward_main_kernel<128>, sizeof(BwdSmem<128>));
  return go(backward_main_kernel<64>, sizeof(BwdSmem<64>));
}

hipError_t launch_backward_postprocess(const msa_problem& p, const void* scratch, void* dq, void* dk,
                                       void* dv, hipStream_t stream) {
  const BackwardScratch L = backward_scratch_layout(p);
  const uint8_t* base = (const uint8_t*)scratch;
  const int64_t hq = (int64_t)p.num_kv_heads * p.q_per_kv;
  const int64_t n_q_vec = (int64_t)p.total_tokens * hq * p.head_dim / 8;
  const int64_t n_kv_vec = (int64_t)p.total_tokens * p.num_kv_heads * p.head_dim / 8;
  const int64_t n = n_q_vec > n_kv_vec ? n_q_vec : n_kv_vec;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(postprocess_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const float*)(base + L.dq_pool), (const float*)(base + L.dk_acc),
                     (const float*)(base + L.dv_acc), (bf16*)dq, (bf16*)dk, (bf16*)dv, n_q_vec, n_kv_vec,
                     p.softmax_scale);
  return hipGetLastError();
}

}  // namespace msa
