// Device helpers shared by the gfx950 kernels of libmsa.
//
// MFMA and LDS-transpose lane layouts used below (CDNA4, wave64):
//  v_mfma_f32_32x32x16_bf16  A (32 x 16): lane l holds row l%32, k = 8*(l/32) + 0..7
//                            B (16 x 32): lane l holds col l%32, k = 8*(l/32) + 0..7
//                            C (32 x 32): lane l, register j holds col l%32,
//                                         row 8*(j/4) + 4*(l/32) + j%4
//  ds_read_tr16_b64          in each 16-lane group g, lane 16g + x receives, as
//                            element r (0..3), 16-bit element x%4 of the 8 bytes
//                            addressed by lane 16g + 4r + x/4.
// An accumulator can feed a later MFMA as an A or B operand directly when the
// contraction runs over its row index: the row order inside a 16-wide k step
// is a permutation, and the other operand is read in the same permuted order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 8;        // queries per chunk
constexpr int kQPerKV = 16;      // query heads per index/KV head
constexpr int kTileM = 128;      // 8 queries x 16 heads
constexpr int kBlock = 64;       // key block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One transposing LDS read of 4 bf16 (see the layout note above).
__device__ __forceinline__ shortx4 lds_read_tr4(const void* lds_ptr) {
  lds_shortx4* p = (lds_shortx4*)(const_cast<void*>(lds_ptr));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

__device__ __forceinline__ bf16x8 join_tr(shortx4 lo, shortx4 hi) {
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  shortx8 s = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, s);
}

// Operand for a K step of 16 along the rows of a row-major [rows][cols] bf16
// tile in LDS (element (r, c) at base + r*ld + c): lane l receives column
// col0 + l%32 and, as elements 0..7, rows
//   row_lo(h) + 0..3 and row_hi(h) + 0..3, h = l/32,
// where the caller passes row_lo/row_hi for its own h.  Used for operands
// whose contraction index is the tile's row index.
__device__ __forceinline__ bf16x8 lds_tr_operand(const bf16* base, int ld, int col0, int lane,
                                                 int row_lo_h0, int row_lo_h1, int row_hi_h0,
                                                 int row_hi_h1) {
  // Source-lane role: this lane supplies the address for group g = lane/16,
  // row r = (lane%16)/4, 4-column chunk c = lane%4.
  const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
  const int h = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * c;
  const int rlo = (h ? row_lo_h1 : row_lo_h0) + r;
  const int rhi = (h ? row_hi_h1 : row_hi_h0) + r;
  shortx4 lo = lds_read_tr4(base + rlo * ld + col);
  shortx4 hi = lds_read_tr4(base + rhi * ld + col);
  return join_tr(lo, hi);
}

__device__ __forceinline__ bf16x8 load_bf16x8_lds(const bf16* p);

// ---------------------------------------------------------------------------
// Unpadded row-major bf16 tiles whose 16-byte chunks are XOR-swizzled per row
// (D = 8 * CPR elements per row).  The swizzle keeps both access patterns of
// the kernels free of LDS bank conflicts on a 64-bank LDS:
//  * 16 consecutive rows read at one logical chunk (MFMA row operands), and
//  * 4 consecutive rows read across 4 consecutive chunks (transpose loads).
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int row) {
  static_assert(CPR == 16 || CPR == 8, "rows of 128 or 64 bf16");
  if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, col) in a swizzled tile with CPR chunks per row.
template <int CPR>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * (8 * CPR) + ((((col >> 3) ^ chunk_swizzle<CPR>(row))) << 3) + (col & 7);
}

// MFMA row operand: 8 consecutive bf16 of `row` starting at col (col % 8 == 0).
template <int CPR>
__device__ __forceinline__ bf16x8 lds_row8(const bf16* tile, int row, int col) {
  return load_bf16x8_lds(tile + swz_off<CPR>(row, col));
}

// Transposing operand from a swizzled tile (same contract as lds_tr_operand).
template <int CPR>
__device__ __forceinline__ bf16x8 lds_tr_operand_swz(const bf16* tile, int col0, int lane, int row_lo_h0,
                                                     int row_lo_h1, int row_hi_h0, int row_hi_h1) {
  const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
  const int h = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * c;
  const int rlo = (h ? row_lo_h1 : row_lo_h0) + r;
  const int rhi = (h ? row_hi_h1 : row_hi_h0) + r;
  shortx4 lo = lds_read_tr4(tile + swz_off<CPR>(rlo, col));
  shortx4 hi = lds_read_tr4(tile + swz_off<CPR>(rhi, col));
  return join_tr(lo, hi);
}

// 64-column bf16 tile (128-byte rows) swizzled in 8-byte slots: slot s of
// row r is stored at slot s ^ p8(r).  Written 8 bytes per lane down 32
// consecutive rows and read with the transpose load (4 rows x 4 slots per
// 16 lanes), both patterns hit every LDS bank once per 32 lanes; a 16-byte
// chunk swizzle leaves the column writes two-way conflicted.
__device__ __forceinline__ int slot_swizzle8(int row) { return ((row >> 1) & 15) ^ ((row & 3) << 2); }
__device__ __forceinline__ int swz8b_off(int row, int col) {
  return row * 64 + (((col >> 2) ^ slot_swizzle8(row)) << 2) + (col & 3);
}
// Transposing operand from such a tile (same contract as lds_tr_operand).
__device__ __forceinline__ bf16x8 lds_tr_operand_swz8b(const bf16* tile, int col0, int lane, int row_lo_h0,
                                                       int row_lo_h1, int row_hi_h0, int row_hi_h1) {
  const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
  const int h = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * c;
  const int rlo = (h ? row_lo_h1 : row_lo_h0) + r;
  const int rhi = (h ? row_hi_h1 : row_hi_h0) + r;
  shortx4 lo = lds_read_tr4(tile + swz8b_off(rlo, col));
  shortx4 hi = lds_read_tr4(tile + swz8b_off(rhi, col));
  return join_tr(lo, hi);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l of the wave writes
// bytes [16 l, 16 l + 16) after lds_wave_base (wave-uniform), reading from a
// wave-uniform base plus the lane's 32-bit byte offset (the buffer form of
// the copy).  The buffer form also keeps the compiler's LDS waits exact:
// the global form is a flat-encoded instruction, and while one is pending
// the compiler waits for every outstanding LDS read (lgkmcnt(0)) wherever it
// needs only the oldest.
__device__ __forceinline__ void dma16_at(const void* sbase, uint32_t byte_off, void* lds_wave_base) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(sbase), (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)byte_off, 0, 0, 0);
}

// Wait until this wave has no outstanding vector-memory operations.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }


__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 load_bf16x8_lds(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_bf16x8(bf16* p, bf16x8 v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}
// Streaming variants (non-temporal hint): data written or read once, kept
// from displacing data that is reused.
__device__ __forceinline__ void store_bf16x8_stream(bf16* p, bf16x8 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ bf16x8 load_bf16x8_stream(const bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void store_bf16x4(bf16* p, bf16x4 v) {
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// The wave's LDS writes are done (and not moved past this point) before its
// later LDS reads; the wave's own LDS accesses execute in order.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding global loads
// and atomics at each barrier; the tiles here share data through LDS only, so
// prefetch loads and fire-and-forget atomics stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for LDS reads and writes made by the waves themselves.  Unlike
// lds_barrier it does not wait for direct global->LDS copies still in flight
// (a release fence on LDS would), so a copy into another buffer keeps going
// across it.  The "memory" clobber keeps the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// K and V rows of one key block in LDS, each an unpadded swizzled tile.
template <int D>
struct KVTiles {
  bf16 k[kBlock * D];
  bf16 v[kBlock * D];
};

// Direct global -> LDS copy of 16 bytes per lane from a per-lane 64-bit
// address, in the global (flat-encoded) form; lane l writes bytes
// [16 l, 16 l + 16) after lds_wave_base.  Only stage_kv uses it: its kernel
// has no registers to spare for the buffer form's descriptors and offsets.
__device__ __forceinline__ void dma16_global(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0,
                                   0);
}

// Copy key block b (K and V rows of KV head i) into a swizzled tile pair with
// 64-bit addresses computed per copy (for kernels with no registers to hold
// precomputed offsets).  Keys past the document end read the document's last
// key instead: they are masked out of the softmax, and their values are finite.
template <int D, int NWAVES>
__device__ __forceinline__ void stage_kv(KVTiles<D>& t, const bf16* __restrict__ k,
                                         const bf16* __restrict__ v, int tok0, int len, int b, int Hkv,
                                         int i, int w, int lane) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPP = 64 / CPR;              // rows per piece
  constexpr int PIECES = kBlock / RPP;       // pieces per tensor
  const int64_t row_stride = (int64_t)Hkv * D;
  const bf16* kbase = k + ((int64_t)tok0 * Hkv + i) * D;
  const bf16* vbase = v + ((int64_t)tok0 * Hkv + i) * D;
  const int lrow = lane / CPR, pcol = lane % CPR;
  const int kmax = len - 1 - b * kBlock;     // last valid key offset in this block
#pragma unroll
  for (int n = 0; n < PIECES / NWAVES; ++n) {
    const int piece = n * NWAVES + w;
    const int row = piece * RPP + lrow;
    const int lc = pcol ^ chunk_swizzle<CPR>(row);
    const int64_t off = (int64_t)(b * kBlock + min(row, kmax)) * row_stride + 8 * lc;
    dma16_global(kbase + off, t.k + piece * 512);
    dma16_global(vbase + off, t.v + piece * 512);
  }
}


// Copy key block b of one tensor (K, say) of KV head i into a swizzled
// kBlock x D tile; 64 / CPR rows per wave-sized piece, keys past the document
// end read the document's last key (masked by the consumer).
template <int D, int NWAVES>
__device__ __forceinline__ void stage_block(bf16* tile, const bf16* __restrict__ src, int tok0, int len,
                                            int b, int Hkv, int i, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPP = 64 / CPR;
  constexpr int N = kBlock / RPP / NWAVES;
  const bf16* first = src + ((int64_t)(tok0 + b * kBlock) * Hkv + i) * D;
  // byte offsets: row * stride does not depend on the block (kept out of the
  // block loop by the compiler), the clamp to the last key is one min.
  const int stride = Hkv * D * 2;
  const int kmax_off = (len - 1 - b * kBlock) * stride;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int piece = n * NWAVES + w;
    const int row = piece * RPP + lane / CPR;
    const int lc = (lane % CPR) ^ chunk_swizzle<CPR>(row);
    const uint32_t o = (uint32_t)(min(row * stride, kmax_off) + 16 * lc);
    dma16_at(first, o, tile + piece * 512);
  }
}

// Kernel tiles hold kBlock = 64 keys; a selected block of `sub` * 64 keys
// (key block 128: sub = 2) is taken as `sub` consecutive 64-key tiles.
// Lane s < sub * K stands for tile `sub * row[s / sub] + s % sub` of slot
// s / sub.  A tile is kept when its slot is kept and its first key is not
// after the chunk's last query `last_q` (later tiles hold only masked keys;
// with sub = 1 every kept slot passes).  Returns the tile id or -1.
__device__ __forceinline__ int sub_tile(const int32_t* __restrict__ row, int K, int sub, int last_q,
                                        int lane) {
  if (lane >= sub * K) return -1;
  const int slot = sub == 1 ? lane : lane >> 1;
  const int b = row[slot];
  const int t = sub * b + (lane - sub * slot);
  return b >= 0 && t * kBlock <= last_q ? t : -1;
}

// Kept tiles of a selection row compacted in lane order: blocks[n] = tile
// id, slots[n] = its position sub * slot + s % sub in the row's tile list.
__device__ __forceinline__ int compact_tiles(const int32_t* __restrict__ row, int K, int sub, int last_q,
                                             int lane, int* blocks, int* slots) {
  const int t = sub_tile(row, K, sub, last_q, lane);
  const bool keep = t >= 0;
  const uint64_t mask = __builtin_amdgcn_ballot_w64(keep);
  const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  if (keep) {
    blocks[pos] = t;
    slots[pos] = lane;
  }
  return __popcll(mask);
}

// acc + sum of the 8 bf16 values of v (dot products with (1, 1) on bf16 pairs).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 pr = {v[2 * e], v[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

// Block-wide inclusive scan of one int per thread (blockDim.x == NT, a
// multiple of 64); s_warp holds NT / 64 ints; *total receives the sum.
template <int NT>
__device__ int block_inclusive_scan_n(int x, int* s_warp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_warp[w] = x;
  __syncthreads();
  int add = 0, tot = 0;
  for (int k = 0; k < NT / 64; ++k) {
    if (k < w) add += s_warp[k];
    tot += s_warp[k];
  }
  __syncthreads();
  *total = tot;
  return x + add;
}

// What a kernel writes instead of its outputs when the schedule's geometry
// check failed (cu_seqlens disagree with the host sizes): NaN in n8 groups of
// 8 bf16 at p and n1 floats at f, grid-stride over every thread of the
// launch.  The sizes come from the host, so the fill stays in bounds
// whatever cu_seqlens hold.
__device__ __forceinline__ void fill_nan(bf16* p, int64_t n8, float* f, int64_t n1) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const u32x4 nan8 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int64_t x = t; x < n8; x += stride) *reinterpret_cast<u32x4*>(p + 8 * x) = nan8;
  for (int64_t x = t; x < n1; x += stride) f[x] = __builtin_nanf("");
}

// Index of the last element <= x in a non-decreasing array a[0..n) (a[0] <= x).
__device__ __forceinline__ int upper_bound_minus1(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace msa
