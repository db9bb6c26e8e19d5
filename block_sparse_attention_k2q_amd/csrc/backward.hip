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
constexpr int kMaxWalk = 64;   // ROWS_PER_CTA_LARGE: longest walk a workgroup takes

// ---------------------------------------------------------------------------
// Preprocess: Delta = rowsum(dO * O) in fp32; zero the dQ pool (fp32 or bf16)
// and dK/dV.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const bf16* __restrict__ out,
                                                         const bf16* __restrict__ dout,
                                                         float* __restrict__ delta,
                                                         float* __restrict__ dq_pool,
                                                         float* __restrict__ dkv, int64_t n_vec,
                                                         int64_t n_dkv_vec, int zero_pool) {
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
  if (zero_pool == 1) {          // fp32 pool: 8 floats per vector
    floatx4* p = reinterpret_cast<floatx4*>(dq_pool) + 2 * x;
    p[0] = floatx4{};
    p[1] = floatx4{};
  } else if (zero_pool == 2) {   // bf16 pool: 8 bf16 per vector
    reinterpret_cast<floatx4*>(dq_pool)[x] = floatx4{};
  }
}

// ---------------------------------------------------------------------------
// Postprocess: dq = bf16(scale * pool), dk = bf16(scale * dk_acc), dv = bf16(dv_acc).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void postprocess_kernel(const float* __restrict__ dq_pool,
                                                          const float* __restrict__ dk_acc,
                                                          const float* __restrict__ dv_acc,
                                                          bf16* __restrict__ dq, bf16* __restrict__ dk,
                                                          bf16* __restrict__ dv, int64_t n_q_vec,
                                                          int64_t n_kv_vec, float scale,
                                                          const int32_t* __restrict__ err) {
  if (err[1]) {   // geometry mismatch: the main kernel did not run
    fill_nan(dq, n_q_vec, nullptr, 0);
    fill_nan(dk, n_kv_vec, nullptr, 0);
    fill_nan(dv, n_kv_vec, nullptr, 0);
    return;
  }
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

// dq from the head-pair-interleaved bf16 pool (already scaled): thread x
// writes dq elements 8x .. 8x+7 = (token, head h, d0 .. d0+7).
template <int D>
__global__ __launch_bounds__(256) void pool_bf16_to_dq_kernel(const bf16* __restrict__ pool,
                                                              bf16* __restrict__ dq, int64_t n_q_vec,
                                                              const int32_t* __restrict__ err) {
  if (err[1]) {
    fill_nan(dq, n_q_vec, nullptr, 0);
    return;
  }
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n_q_vec) return;
  const int64_t e = 8 * x;
  const int d0 = (int)(e % D);
  const int64_t th = e / D;                 // token * Hq + h
  const int64_t pair = th >> 1, odd = th & 1;
  const bf16x8 a = load_bf16x8(pool + (pair * D + d0) * 2);
  const bf16x8 b = load_bf16x8(pool + (pair * D + d0) * 2 + 8);
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = a[2 * k + odd];
    r[4 + k] = b[2 * k + odd];
  }
  store_bf16x8(dq + e, r);
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
  int meta[kMaxWalk][9];   // per walked task: i, r, qb, qc, d, b, tok0, len, first K/V row of d
};

template <int D, bool BF16_POOL>
__global__ __launch_bounds__(kBwdThreads, 1) void backward_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ task_meta,
    const int32_t* __restrict__ desc, const int32_t* __restrict__ err, void* __restrict__ dq_pool,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, const int32_t* __restrict__ doc_kv_off, int Hkv,
    int sub, float scale) {
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
  // Key block 128 (sub = 2): workgroup 2x + kt takes the 64-key half kt of
  // every task of walk x.
  const int wg = blockIdx.x / sub;
  const int kt = blockIdx.x % sub;
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

  int cur_i = -1, cur_r = -1, cur_kv0 = 0, cur_len = 0, cur_b = 0;

  auto flush = [&]() {
#pragma unroll
    for (int x = 0; x < OUT_TILES; ++x) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // Keys past the document end hold exact zeros (zero K/V rows, masked
        // P); they are sent to the block's first key so the atomics need no branch.
        const int key = 32 * own_mt[x] + 8 * (j >> 2) + 4 * h + (j & 3);
        const int kpos = cur_b * kBlock + (cur_b * kBlock + key < cur_len ? key : 0);
        const int64_t off = ((int64_t)(cur_kv0 + kpos) * Hkv + cur_i) * D + 32 * own_nt[x] + n32;
        atomicAdd(dv_acc + off, acc_dv[x][j]);
        atomicAdd(dk_acc + off, acc_dk[x][j]);
      }
    }
  };

  // The walk's task rows, with their document start and length, once into LDS.
  const int nrows = hi - lo;
  for (int e = threadIdx.x; e < nrows; e += kBwdThreads) {
    const int32_t* tm = task_meta + (int64_t)(lo + e) * 6;
    int* m = sm.meta[e];
#pragma unroll
    for (int x = 0; x < 6; ++x) m[x] = tm[x];
    m[5] = sub * tm[5] + kt;     // the task's 64-key tile
    const int d = tm[4];
    const int t0 = cu[d];
    m[6] = t0;
    m[7] = cu[d + 1] - t0;
    m[8] = doc_kv_off[d];
  }
  lds_barrier();

  // Register prefetch of one tile: Q and dO rows (m = token * 16 + head; zero
  // past the document end) and the raw LSE (threads 0..127) or Delta
  // (threads 128..255) of row m.  Nothing here consumes the loaded values, so
  // the loads stay in flight while the current tile computes.
  constexpr int PFV = kTileM * VEC / kBwdThreads;
  u32x4 pq_[PFV], po_[PFV];
  float pscal = 0.f;
  const bool is_lse_thread = threadIdx.x < kTileM;
  auto prefetch = [&](int e) {
    const int* m = sm.meta[e];
    const int i = m[0], qb = m[2], qc = m[3], tok0 = m[6];
#pragma unroll
    for (int x = 0; x < PFV; ++x) {
      const int idx = threadIdx.x + x * kBwdThreads;
      const int mm = idx / VEC, col = (idx % VEC) * 8;
      const int j = mm >> 4, hh = mm & 15;
      if (j < qc) {
        const int64_t off = ((int64_t)(tok0 + qb + j) * Hq + kQPerKV * i + hh) * D + col;
        pq_[x] = *reinterpret_cast<const u32x4*>(q + off);
        po_[x] = *reinterpret_cast<const u32x4*>(dout + off);
      } else {
        pq_[x] = u32x4{0, 0, 0, 0};
        po_[x] = u32x4{0, 0, 0, 0};
      }
    }
    const int mm = threadIdx.x & (kTileM - 1), j = mm >> 4, hh = mm & 15;
    const int64_t rowi = (int64_t)(tok0 + qb + min(j, qc - 1)) * Hq + kQPerKV * i + hh;
    pscal = is_lse_thread ? lse[rowi] : delta[rowi];
  };
  if (nrows > 0) prefetch(0);

  for (int row = lo; row < hi; ++row) {
    const int* mrow = sm.meta[row - lo];
    const int i = mrow[0], r = mrow[1], qb = mrow[2], qc = mrow[3], b = mrow[5];
    const int tok0 = mrow[6], len = mrow[7], kv0 = mrow[8];
    lds_barrier();  // previous tile fully consumed
    if (i != cur_i || r != cur_r) {
      // a half tile that starts past the document end holds no key
      if (cur_i >= 0 && cur_b * kBlock < cur_len) flush();
#pragma unroll
      for (int x = 0; x < OUT_TILES; ++x) {
        acc_dv[x] = floatx16{};
        acc_dk[x] = floatx16{};
      }
      cur_i = i; cur_r = r; cur_kv0 = kv0; cur_len = len; cur_b = b;
      for (int e = threadIdx.x; e < kBlock * VEC; e += kBwdThreads) {
        const int kr = e / VEC, col = (e % VEC) * 8;
        const int kpos = b * kBlock + kr;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (kpos < len) {
          const int64_t off = ((int64_t)(kv0 + kpos) * Hkv + i) * D + col;
          kv = *reinterpret_cast<const u32x4*>(k + off);
          vv = *reinterpret_cast<const u32x4*>(v + off);
        }
        *reinterpret_cast<u32x4*>(&sm.k[kr * LDK + col]) = kv;
        *reinterpret_cast<u32x4*>(&sm.v[kr * LDK + col]) = vv;
      }
    }
#pragma unroll
    for (int x = 0; x < PFV; ++x) {
      const int idx = threadIdx.x + x * kBwdThreads;
      const int mm = idx / VEC, col = (idx % VEC) * 8;
      *reinterpret_cast<u32x4*>(&sm.q[mm * LDK + col]) = pq_[x];
      *reinterpret_cast<u32x4*>(&sm.dout[mm * LDK + col]) = po_[x];
    }
    {
      // Rows past the document end get LSE = +inf (so P = 0) and Delta = 0.
      const int mm = threadIdx.x & (kTileM - 1);
      const bool valid = (mm >> 4) < qc;
      if (is_lse_thread)
        sm.lse2[mm] = (valid && pscal != -INFINITY) ? pscal * kLog2e : INFINITY;
      else
        sm.delta[mm] = valid ? pscal : 0.f;
    }
    lds_barrier();
    if (row + 1 < hi) prefetch(row + 1 - lo);

    // --- S^T and dP^T for this wave's 32 query rows -------------------------
    // Operands of k step s+1 are read from LDS while step s runs on the MFMA.
    const int mq = 32 * w + n32;   // this lane's query row in the tile
    floatx16 st[2] = {floatx16{}, floatx16{}};
    floatx16 dpt[2] = {floatx16{}, floatx16{}};
    {
      bf16x8 bq[2], bo[2], ak[2][2], av[2][2];
      auto load_step = [&](int s, int slot) {
        bq[slot] = load_bf16x8(&sm.q[mq * LDK + 16 * s + 8 * h]);
        bo[slot] = load_bf16x8(&sm.dout[mq * LDK + 16 * s + 8 * h]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ak[slot][t] = load_bf16x8(&sm.k[(32 * t + n32) * LDK + 16 * s + 8 * h]);
          av[slot][t] = load_bf16x8(&sm.v[(32 * t + n32) * LDK + 16 * s + 8 * h]);
        }
      };
      load_step(0, 0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) load_step(s + 1, (s + 1) & 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          st[t] = mfma32(ak[s & 1][t], bq[s & 1], st[t]);
          dpt[t] = mfma32(av[s & 1][t], bo[s & 1], dpt[t]);
        }
      }
    }
    const float l2 = sm.lse2[mq];
    const float dl = sm.delta[mq];
    // Only the diagonal block holds keys after a query (or past the document
    // end): there, keys at block offset > klim get score -inf, so P = 0.
    if ((b + 1) * kBlock - 1 > qb) {
      const int pq = qb + (mq >> 4);
      const int klim = min(pq, len - 1) - b * kBlock;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = 32 * t + 8 * (j >> 2) + 4 * h + (j & 3);
          st[t][j] = key <= klim ? st[t][j] : -INFINITY;
        }
    }
    bf16x8 dsa[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4 p4, d4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int j = 4 * jg + rr;
          const float pv = fast_exp2(fmaf(st[t][j], c2, -l2));
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

    // --- dQ = dS K (32 query rows x D) -> dQ pool ------------------------------
    {
      floatx16 dq[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) dq[t] = floatx16{};
      bf16x8 bk[2][NT];
      auto load_k = [&](int u, int slot) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          bk[slot][t] = lds_tr_operand(sm.k, LDK, 32 * t, lane, 16 * u, 16 * u + 4, 16 * u + 8,
                                       16 * u + 12);
      };
      load_k(0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u + 1 < 4) load_k(u + 1, (u + 1) & 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) dq[t] = mfma32(dsa[u], bk[u & 1][t], dq[t]);
      }
      // Accumulator: column = d (lane), rows = query rows 8(j/4) + 4h + j%4 of
      // this wave.  Rows past the document end hold exact zeros (their P and
      // dS are 0); they are sent to the tile's first row, which always exists,
      // so the atomics need no branch.
      const int64_t row0 = (int64_t)(tok0 + qb) * Hq + kQPerKV * i;
      if constexpr (BF16_POOL) {
        // Registers j and j+1 (j even) hold heads hh and hh+1 of one token:
        // one packed atomic adds both, pre-scaled, into the interleaved pool.
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const int64_t pair0 = row0 >> 1;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const int m = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
          const int jt = m >> 4, hh = m & 15;
          const int64_t pr = jt < qc ? pair0 + (int64_t)jt * (Hq / 2) + (hh >> 1) : pair0;
          bf16x2* dst = reinterpret_cast<bf16x2*>(dq_pool) + pr * D + n32;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16x2 val = {(bf16)(dq[t][j] * scale), (bf16)(dq[t][j + 1] * scale)};
            __builtin_amdgcn_global_atomic_fadd_v2bf16(
                (__attribute__((address_space(1))) bf16x2*)(dst + 32 * t), val);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
          const int jt = m >> 4, hh = m & 15;
          const int64_t rowm = jt < qc ? row0 + (int64_t)jt * Hq + hh : row0;
          float* dst = reinterpret_cast<float*>(dq_pool) + rowm * D + n32;
#pragma unroll
          for (int t = 0; t < NT; ++t) atomicAdd(dst + 32 * t, dq[t][j]);
        }
      }
    }
    lds_barrier();  // P, dS complete in LDS

    // --- dV += P^T dO, dK += dS^T Q over all 128 query rows -------------------
    {
      bf16x8 ap[2][OUT_TILES], ad[2][OUT_TILES], bo[2][OUT_TILES], bq[2][OUT_TILES];
      auto load_u = [&](int u, int slot) {
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x) {
          const int mt = own_mt[x], nt = own_nt[x];
          ap[slot][x] = lds_tr_operand(sm.p, LDP, 32 * mt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                       16 * u + 12);
          bo[slot][x] = lds_tr_operand(sm.dout, LDK, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                       16 * u + 12);
          ad[slot][x] = lds_tr_operand(sm.ds, LDP, 32 * mt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                       16 * u + 12);
          bq[slot][x] = lds_tr_operand(sm.q, LDK, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                       16 * u + 12);
        }
      };
      load_u(0, 0);
#pragma unroll
      for (int u = 0; u < kTileM / 16; ++u) {
        if (u + 1 < kTileM / 16) load_u(u + 1, (u + 1) & 1);
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x) {
          acc_dv[x] = mfma32(ap[u & 1][x], bo[u & 1][x], acc_dv[x]);
          acc_dk[x] = mfma32(ad[u & 1][x], bq[u & 1][x], acc_dk[x]);
        }
      }
    }
  }
  if (cur_i >= 0 && cur_b * kBlock < cur_len) flush();
}

// ---------------------------------------------------------------------------
// Main kernel of the MSA_DQ_RECOMPUTE mode: S^T, dP^T, dV, dK only.
//
// Two workgroups share each walk: workgroup 2x + half takes query rows
// 64*half .. 64*half + 63 (tokens 4*half .. 4*half + 3 of the chunk, all 16
// heads of the index head) of every task tile of walk x and accumulates its
// own partial dK / dV of the bucket.  Each workgroup then needs under 80 KB
// of LDS and under 256 registers per lane, so two run on every CU and the
// softmax arithmetic of one overlaps the matrix-core work of the other.
//
//  * wave w handles queries 32*(w & 1) .. +31 of the half against keys
//    32*(w >> 1) .. +31 of the block: K and V of those keys live in
//    registers as the A operands of S^T = K Q^T and dP^T = V dO^T (loaded
//    once per bucket segment), each lane owning one query column;
//  * the Q and dO rows of the half arrive in LDS by direct global->LDS
//    loads into one of two swizzled buffers, the next task's copy in flight
//    while the current one is consumed (each lane's LSE and Delta are loaded
//    into registers one task ahead);
//  * P^T goes to an LDS tile for dV += P^T dO, then dS^T (kept in
//    registers meanwhile) overwrites it for dK += dS^T Q; each wave owns
//    2 (head dim 128) or 1 (head dim 64) of the 32 x 32 output tiles of dV
//    and of dK.
//
// Key block 128 (KT = 2 key tiles of 64): one workgroup of 8 waves per walk
// half, waves 4t .. 4t+3 doing the above for keys 64t .. 64t+63 of the
// block, so both halves of the block share one gather of the Q / dO rows
// (msa_schedule page: BLOCK_SIZE 128; msa_backward_sm100 page: TILE_N 128).
// ---------------------------------------------------------------------------
constexpr int kHalfM = kTileM / 2;

template <int D>
struct KvHalf {
  bf16 q[kHalfM * D];
  bf16 dout[kHalfM * D];
};

// Copy the Q / dO rows of one half task tile into a swizzled buffer.  Rows
// past the document end read the chunk's last valid row (their
// probabilities are forced to 0 by the consumer).
template <int D, int NW>
__device__ __forceinline__ void stage_qdo(KvHalf<D>& t, const bf16* __restrict__ q,
                                          const bf16* __restrict__ dout, const int* m, int half, int Hq,
                                          int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPP = 64 / CPR;                 // rows per wave-sized piece
  constexpr int PIECES = kHalfM / RPP;          // pieces per tensor
  static_assert(PIECES % NW == 0 && 16 % RPP == 0, "pieces split evenly over the waves, within a token");
  const int i = __builtin_amdgcn_readfirstlane(m[0]), qb = __builtin_amdgcn_readfirstlane(m[2]);
  const int qc = __builtin_amdgcn_readfirstlane(m[3]), tok0 = __builtin_amdgcn_readfirstlane(m[6]);
  const int lrow = lane / CPR, pcol = lane % CPR;
#pragma unroll
  for (int n = 0; n < PIECES / NW; ++n) {
    const int piece = n * NW + w;
    const int row = piece * RPP + lrow;         // local row = (token - 4*half) * 16 + head
    // all rows of a piece belong to one token: a wave-uniform base per piece
    const int j = min(4 * half + ((piece * RPP) >> 4), qc - 1);
    const int64_t first = ((int64_t)(tok0 + qb + j) * Hq + kQPerKV * i) * D;
    const int lc = pcol ^ chunk_swizzle<CPR>(row);
    const uint32_t off = (uint32_t)((row & 15) * D + 8 * lc) * 2u;
    dma16_at(q + first, off, t.q + piece * 512);
    dma16_at(dout + first, off, t.dout + piece * 512);
  }
}

template <int D, bool WRITE_DS, int KT>
__global__ __launch_bounds__(kBwdThreads * KT, 2 / KT) void backward_kv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ task_meta,
    const int32_t* __restrict__ desc, const int32_t* __restrict__ err, float* __restrict__ dk_acc,
    float* __restrict__ dv_acc, bf16* __restrict__ ds, const int32_t* __restrict__ doc_chunk_off,
    const int32_t* __restrict__ doc_kv_off, const int32_t* __restrict__ sel_clean, int Hkv, int C, int K,
    int sub, float scale) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;
  constexpr int NT = D / 32;
  constexpr int OUT_TILES = 2 * NT / 4;        // dV (and dK) output tiles per wave
  static_assert(NT == 4 || NT == 2, "head dim 128 or 64");
  static_assert(KT == 1 || KT == 2, "one or two 64-key tiles per workgroup");
  constexpr int NW = 4 * KT;                   // waves
  // Separate objects, so the compiler can tell the copy into one buffer
  // from reads of the other (and of pd) and waits only where needed.
  __shared__ __attribute__((aligned(16))) KvHalf<D> tile0;
  __shared__ __attribute__((aligned(16))) KvHalf<D> tile1;
  // P^T, then dS^T, of each key tile (rows = queries)
  __shared__ __attribute__((aligned(16))) bf16 pd_all[KT][kHalfM * kBlock];
  // per walked task: i, r, qb, qc, dS slot of the first tile, first tile, tok0, len,
  // first K/V row of the document
  __shared__ int meta[kMaxWalk][9];

  if (err[1]) return;
  const int grid_walks = desc[5];
  // Workgroup 2x + half takes query half `half` of every task of walk x.
  const int wg = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
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
  const int kt = KT == 1 ? 0 : w >> 2;         // this wave's 64-key tile of the block
  const int wl = KT == 1 ? w : w & 3;          // its wave within that tile
  bf16* const pd = pd_all[kt];
  const int n32 = lane & 31, h = lane >> 5;
  const int Hq = Hkv * kQPerKV;
  const float c2 = scale * kLog2e;
  const int mq = 32 * (wl & 1) + n32;          // this lane's query row in the half tile
  const int kh = wl >> 1;                      // this wave's 32-key half of the tile
  const int jtok = 4 * half + (mq >> 4);       // its token within the chunk

  int own_mt[OUT_TILES], own_nt[OUT_TILES];
#pragma unroll
  for (int x = 0; x < OUT_TILES; ++x) {
    const int tile = wl * OUT_TILES + x;
    own_nt[x] = tile / 2;
    own_mt[x] = tile % 2;
  }
  floatx16 acc_dv[OUT_TILES], acc_dk[OUT_TILES];
  bf16x8 ka[KS], va[KS];                       // K, V rows of this wave's keys as MFMA A operands
  int cur_i = -1, cur_r = -1, cur_kv0 = 0, cur_len = 0, cur_b = 0;

  auto flush = [&]() {
    // Partial dK/dV of the finished bucket segment; keys past the document
    // end hold exact zeros and are sent to the block's first key.  Register
    // j of tile x holds key 32 mt + 4h + c_j, c_j = 8(j/4) + j%4.
    const int stride = Hkv * D;
#pragma unroll
    for (int x = 0; x < OUT_TILES; ++x) {
      int kb = 32 * own_mt[x] + 4 * h;
      asm volatile("" : "+v"(kb));   // keep the per-register offsets below out of the task loop
      const int64_t first = ((int64_t)(cur_kv0 + cur_b * kBlock) * Hkv + cur_i) * D + 32 * own_nt[x] + n32;
      float* dvp = dv_acc + first;
      float* dkp = dk_acc + first;
      const int room = cur_len - cur_b * kBlock - kb;   // c_j < room: key inside the document
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = 8 * (j >> 2) + (j & 3);
        const int rel = c < room ? (kb + c) * stride : 0;
        atomicAdd(dvp + rel, acc_dv[x][j]);
        atomicAdd(dkp + rel, acc_dk[x][j]);
      }
    }
  };

  const int nrows = hi - lo;
  for (int e = threadIdx.x; e < nrows; e += kBwdThreads * KT) {
    const int32_t* tm = task_meta + (int64_t)(lo + e) * 6;
    int* m = meta[e];
#pragma unroll
    for (int x = 0; x < 6; ++x) m[x] = tm[x];
    m[5] = sub * tm[5];          // the block's first 64-key tile (a wave adds its kt)
    const int d = tm[4];
    const int t0 = cu[d];
    m[6] = t0;
    m[7] = cu[d + 1] - t0;
    m[8] = doc_kv_off[d];
    if constexpr (WRITE_DS) {
      // dS slot of the tile: (index head, global chunk, position of its block
      // in the chunk's cleaned selection, tile); the document id is not
      // needed later.
      const int64_t row = (int64_t)tm[0] * C + doc_chunk_off[d] + tm[2] / kChunk;
      const int32_t* sel = sel_clean + row * K;
      int slot = -1;
      for (int x = 0; x < K; ++x) slot = sel[x] == tm[5] ? x : slot;
      m[4] = slot < 0 ? -1 : (int)((row * K + slot) * sub);   // first tile's slot
    }
  }
  lds_barrier();
  // LSE and Delta of this lane's query row, fetched one task ahead.
  auto row_index = [&](const int* m) {
    return (int64_t)(m[6] + m[2] + min(jtok, m[3] - 1)) * Hq + kQPerKV * m[0] + (mq & 15);
  };
  float next_lse = 0.f, next_delta = 0.f;
  if (nrows > 0) {
    stage_qdo<D, NW>(tile0, q, dout, meta[0], half, Hq, w, lane);
    next_lse = lse[row_index(meta[0])];
    next_delta = delta[row_index(meta[0])];
  }

  // One task: T holds its half tile, N receives the next task's.
  auto step = [&](int row, KvHalf<D>& T, KvHalf<D>& N) {
    const int e = row - lo;
    const int* mrow = meta[e];
    // wave-uniform task fields, kept in scalar registers
    const int i = __builtin_amdgcn_readfirstlane(mrow[0]), r = __builtin_amdgcn_readfirstlane(mrow[1]);
    const int qb = __builtin_amdgcn_readfirstlane(mrow[2]), qc = __builtin_amdgcn_readfirstlane(mrow[3]);
    const int b = __builtin_amdgcn_readfirstlane(mrow[5]) + kt;
    const int len = __builtin_amdgcn_readfirstlane(mrow[7]);
    const int kv0 = __builtin_amdgcn_readfirstlane(mrow[8]);
    wait_vmem();
    lds_barrier();   // task e landed; every wave is done with task e-1 and with pd

    if (i != cur_i || r != cur_r) {
      if (cur_i >= 0 && cur_b * kBlock < cur_len) flush();   // a tile past the end holds no key
#pragma unroll
      for (int x = 0; x < OUT_TILES; ++x) {
        acc_dv[x] = floatx16{};
        acc_dk[x] = floatx16{};
      }
      cur_i = i; cur_r = r; cur_kv0 = kv0; cur_len = len; cur_b = b;
      // K, V row 32*kh + n32 of the block, d = 16s + 8h .. +7 (keys past the
      // document end read its last key; they are masked).
      const int key = min(b * kBlock + 32 * kh + n32, len - 1);
      const int64_t off = ((int64_t)(kv0 + key) * Hkv + i) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = load_bf16x8(k + off + 16 * s);
        va[s] = load_bf16x8(v + off + 16 * s);
      }
      // Wait here, before the next task's copy is issued: a wait placed by
      // the compiler at the first use would also wait for that copy.
      wait_vmem();
    }
    const float lv = next_lse, dl = next_delta;
    if (row + 1 < hi) {
      stage_qdo<D, NW>(N, q, dout, meta[e + 1], half, Hq, w, lane);
      next_lse = lse[row_index(meta[e + 1])];
      next_delta = delta[row_index(meta[e + 1])];
    }
    // this half holds no token of the chunk (the same for every wave)
    if (4 * half >= qc) return;
    // this wave's tile starts after the chunk's last query (the second tile
    // of a 128-key block: all keys masked); with one tile per workgroup it
    // never happens (the selection keeps only blocks that start by then).
    // The waves of the other tile go on, so the three barriers below are
    // kept here.
    if (b * kBlock > qb + qc - 1) {
      lds_sync();
      lds_sync();
      lds_sync();
      return;
    }

    // --- S^T and dP^T: 32 keys x 32 queries per wave ---------------------------
    floatx16 st = floatx16{}, dpt = floatx16{};
    {
      // Q / dO operands two k steps ahead: one step (two MFMAs) does not
      // cover the LDS latency.
      bf16x8 bq[3], bo[3];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bq[s] = lds_row8<CPR>(T.q, mq, 16 * s + 8 * h);
        bo[s] = lds_row8<CPR>(T.dout, mq, 16 * s + 8 * h);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 2 < KS) {
          bq[(s + 2) % 3] = lds_row8<CPR>(T.q, mq, 16 * (s + 2) + 8 * h);
          bo[(s + 2) % 3] = lds_row8<CPR>(T.dout, mq, 16 * (s + 2) + 8 * h);
        }
        __builtin_amdgcn_sched_barrier(0);
        st = mfma32(ka[s], bq[s % 3], st);
        dpt = mfma32(va[s], bo[s % 3], dpt);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Rows past the document end: LSE = +inf, so P = 0 (and dS = 0).
    const float l2 = (jtok < qc && lv != -INFINITY) ? lv * kLog2e : INFINITY;
    // Only the diagonal block holds keys after a query (or past the document
    // end): there, keys at block offset > klim get score -inf, so P = 0.
    if ((b + 1) * kBlock - 1 > qb) {
      // key offset of register j: 32kh + 4h + 8(j/4) + j%4
      const int klim = min(qb + jtok, len - 1) - b * kBlock - 32 * kh - 4 * h;
#pragma unroll
      for (int j = 0; j < 16; ++j) st[j] = 8 * (j >> 2) + (j & 3) <= klim ? st[j] : -INFINITY;
    }
    bf16x4 ds4[4];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 p4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j = 4 * jg + rr;
        const float pv = fast_exp2(fmaf(st[j], c2, -l2));
        p4[rr] = (bf16)pv;
        ds4[jg][rr] = (bf16)(pv * (dpt[j] - dl));
      }
      // P row of this query, keys 32kh + 8jg + 4h .. +3
      store_bf16x4(pd + swz8b_off(mq, 32 * kh + 8 * jg + 4 * h), p4);
    }
    if constexpr (WRITE_DS) {
      // A slot holds dS in the MFMA operand order of the dQ kernel: for each
      // 32-row block r of the tile and 16-key step u, 64 lanes x 8 bf16, lane
      // n + 32h' carrying row 32r + n, keys 16u + {0..3, 8..11} (h' = 0) or
      // 16u + {4..7, 12..15} (h' = 1).  This lane's row block is
      // 2 half + (wl & 1), its steps 2kh and 2kh + 1, and h' = h.
      const int slot0 = __builtin_amdgcn_readfirstlane(mrow[4]);
      if (slot0 >= 0) {
        const int slot = slot0 + kt;
        bf16* dst = ds + (int64_t)slot * (kDsSlotBytes / 2) +
                    ((2 * half + (wl & 1)) * 4 + 2 * kh) * 512 + lane * 8;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 v8;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v8[r] = ds4[2 * t][r];
            v8[4 + r] = ds4[2 * t + 1][r];
          }
          store_bf16x8_stream(dst + 512 * t, v8);
        }
      }
    }
    lds_sync();      // P complete

    // --- dV += P^T dO over the 64 query rows of the half ------------------------
    {
      const int nt = own_nt[0];
      bf16x8 ap[2][OUT_TILES], bo[2];
      auto load_u = [&](int u, int slot) {
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x)
          ap[slot][x] = lds_tr_operand_swz8b(pd, 32 * own_mt[x], lane, 16 * u, 16 * u + 8,
                                              16 * u + 4, 16 * u + 12);
        bo[slot] = lds_tr_operand_swz<CPR>(T.dout, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                           16 * u + 12);
      };
      load_u(0, 0);
#pragma unroll
      for (int u = 0; u < kHalfM / 16; ++u) {
        if (u + 1 < kHalfM / 16) load_u(u + 1, (u + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x) acc_dv[x] = mfma32(ap[u & 1][x], bo[u & 1], acc_dv[x]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_sync();      // every wave is done reading P
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) store_bf16x4(pd + swz8b_off(mq, 32 * kh + 8 * jg + 4 * h), ds4[jg]);
    lds_sync();      // dS complete

    // --- dK += dS^T Q over the 64 query rows of the half ------------------------
    {
      const int nt = own_nt[0];
      bf16x8 ad[2][OUT_TILES], bq[2];
      auto load_u = [&](int u, int slot) {
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x)
          ad[slot][x] = lds_tr_operand_swz8b(pd, 32 * own_mt[x], lane, 16 * u, 16 * u + 8,
                                              16 * u + 4, 16 * u + 12);
        bq[slot] = lds_tr_operand_swz<CPR>(T.q, 32 * nt, lane, 16 * u, 16 * u + 8, 16 * u + 4,
                                           16 * u + 12);
      };
      load_u(0, 0);
#pragma unroll
      for (int u = 0; u < kHalfM / 16; ++u) {
        if (u + 1 < kHalfM / 16) load_u(u + 1, (u + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < OUT_TILES; ++x) acc_dk[x] = mfma32(ad[u & 1][x], bq[u & 1], acc_dk[x]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int row = lo; row < hi; row += 2) {
    step(row, tile0, tile1);
    if (row + 1 < hi) step(row + 1, tile1, tile0);
  }
  if (cur_i >= 0 && cur_b * kBlock < cur_len) flush();
}

}  // namespace

hipError_t launch_backward_preprocess(const msa_problem& p, const void* out, const void* dout,
                                      void* scratch, hipStream_t stream) {
  const BackwardScratch L = backward_scratch_layout(p);
  uint8_t* base = (uint8_t*)scratch;
  const int64_t hq = (int64_t)p.num_kv_heads * p.q_per_kv;
  const int64_t n_vec = (int64_t)p.total_tokens * hq * p.head_dim / 8;
  // dK and dV accumulators are adjacent: zero both as one range.
  const int64_t n_dkv_vec = (int64_t)(L.dq_pool - L.dk_acc) / 32;
  const int64_t n = n_vec > n_dkv_vec ? n_vec : n_dkv_vec;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, (const bf16*)out, (const bf16*)dout,
                       (float*)(base + L.delta), (float*)(base + L.dq_pool), (float*)(base + L.dk_acc),
                       n_vec, n_dkv_vec,
                       p.dq_mode == MSA_DQ_ATOMIC_POOL ? 1 : p.dq_mode == MSA_DQ_ATOMIC_POOL_BF16 ? 2 : 0);
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
  const int sub = p.block_size / kBlock;
  auto go = [&](auto kern, size_t lds) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(sub * grid)), dim3(kBwdThreads), lds, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                       (const float*)(base + S.delta), cu, sched + L.task_meta, sched + L.desc,
                       sched + L.err, (void*)(base + S.dq_pool), (float*)(base + S.dk_acc),
                       (float*)(base + S.dv_acc), sched + L.doc_kv_off, p.num_kv_heads, sub, p.softmax_scale);
    return hipGetLastError();
  };
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL) {
    if (p.head_dim == 128) return go(backward_main_kernel<128, false>, sizeof(BwdSmem<128>));
    return go(backward_main_kernel<64, false>, sizeof(BwdSmem<64>));
  }
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL_BF16) {
    if (p.head_dim == 128) return go(backward_main_kernel<128, true>, sizeof(BwdSmem<128>));
    return go(backward_main_kernel<64, true>, sizeof(BwdSmem<64>));
  }
  // Two workgroups per walk, one per query half of every task tile; with
  // key block 128 each holds both 64-key tiles of the block (8 waves).
  auto go_kv = [&](auto kern, int kt) {
    hipLaunchKernelGGL(kern, dim3((unsigned)(2 * grid)), dim3(kBwdThreads * kt), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                       (const float*)(base + S.delta), cu, sched + L.task_meta, sched + L.desc,
                       sched + L.err, (float*)(base + S.dk_acc), (float*)(base + S.dv_acc),
                       (bf16*)(base + S.ds), sched + L.doc_chunk_off, sched + L.doc_kv_off, sched + L.sel_clean,
                       p.num_kv_heads, p.num_chunks, p.topk, sub, p.softmax_scale);
    return hipGetLastError();
  };
  if (p.block_size == 128) {
    if (p.dq_mode == MSA_DQ_DS_BUFFER) {
      if (p.head_dim == 128) return go_kv(backward_kv_kernel<128, true, 2>, 2);
      return go_kv(backward_kv_kernel<64, true, 2>, 2);
    }
    if (p.head_dim == 128) return go_kv(backward_kv_kernel<128, false, 2>, 2);
    return go_kv(backward_kv_kernel<64, false, 2>, 2);
  }
  if (p.dq_mode == MSA_DQ_DS_BUFFER) {
    if (p.head_dim == 128) return go_kv(backward_kv_kernel<128, true, 1>, 1);
    return go_kv(backward_kv_kernel<64, true, 1>, 1);
  }
  if (p.head_dim == 128) return go_kv(backward_kv_kernel<128, false, 1>, 1);
  return go_kv(backward_kv_kernel<64, false, 1>, 1);
}

hipError_t launch_backward_postprocess(const msa_problem& p, const int32_t* sched,
                                       const msa_schedule_layout& S, const void* scratch, void* dq, void* dk,
                                       void* dv, hipStream_t stream) {
  const BackwardScratch L = backward_scratch_layout(p);
  const uint8_t* base = (const uint8_t*)scratch;
  const int64_t hq = (int64_t)p.num_kv_heads * p.q_per_kv;
  const int64_t n_q_vec =
      p.dq_mode == MSA_DQ_ATOMIC_POOL ? (int64_t)p.total_tokens * hq * p.head_dim / 8 : 0;
  const int64_t n_kv_vec = kv_rows_of(p) * p.num_kv_heads * p.head_dim / 8;
  const int64_t n = n_q_vec > n_kv_vec ? n_q_vec : n_kv_vec;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(postprocess_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const float*)(base + L.dq_pool), (const float*)(base + L.dk_acc),
                     (const float*)(base + L.dv_acc), (bf16*)dq, (bf16*)dk, (bf16*)dv, n_q_vec, n_kv_vec,
                     p.softmax_scale, sched + S.err);
  if (p.dq_mode == MSA_DQ_ATOMIC_POOL_BF16) {
    const int64_t n_pool_vec = (int64_t)p.total_tokens * hq * p.head_dim / 8;
    if (n_pool_vec > 0) {
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)((n_pool_vec + 255) / 256)), dim3(256), 0, stream,
                           (const bf16*)(base + L.dq_pool), (bf16*)dq, n_pool_vec, sched + S.err);
      };
      if (p.head_dim == 128) go(pool_bf16_to_dq_kernel<128>);
      else go(pool_bf16_to_dq_kernel<64>);
    }
  }
  return hipGetLastError();
}

}  // namespace msa
