// C-ABI entry points of libmsa (declared in include/msa.h).
//
// Host-side checks run before anything is enqueued; kernels only read sizes
// that passed them.  The device gate and the compute-unit count are looked up
// once per device and cached (kernels page: sm_capability / sm_count are
// memoised because the query is paid on every forward).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "msa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
int32_t g_dev_cus[kMaxDevices];

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_problem(const msa_problem* p) {
  if (!p) return MSA_ERR_INVALID;
  if (p->total_tokens < 0 || p->num_docs < 1 || p->num_kv_heads < 1 || p->topk < 1 ||
      p->num_chunks < 0 || p->num_kblocks < 0 || p->max_doc_chunks < 0 || p->num_cus < 1 ||
      p->kv_rows < 0)
    return MSA_ERR_INVALID;
  if (p->q_per_kv != 16 || (p->block_size != 64 && p->block_size != 128) || p->query_chunk != 8 ||
      (p->head_dim != 64 && p->head_dim != 128) || p->topk > 64 ||
      p->max_doc_chunks > MSA_MAX_DOC_CHUNKS)
    return MSA_ERR_UNSUPPORTED;
  // Key block 128 runs as two 64-key halves: at most 64 halves per
  // selection row (one per lane of the wave that compacts the row).
  if (p->block_size == 128 && p->topk > 32) return MSA_ERR_UNSUPPORTED;
  // Size limits so every flat index fits the 32/64-bit arithmetic the kernels use.
  const int64_t cap = (int64_t)p->num_kv_heads * p->num_chunks * p->topk;
  if (cap > (int64_t)INT32_MAX / 6 || (int64_t)p->num_kv_heads * (p->num_kblocks + 1) > INT32_MAX)
    return MSA_ERR_UNSUPPORTED;
  // Geometry implied by the sizes themselves.
  if ((int64_t)p->num_chunks * 8 < p->total_tokens || (int64_t)p->num_kblocks * p->block_size < p->total_tokens ||
      p->num_chunks > p->total_tokens || p->num_kblocks > p->num_chunks ||
      p->max_doc_chunks > p->num_chunks || (p->num_chunks > 0 && p->max_doc_chunks < 1) ||
      (p->kv_rows > 0 && p->kv_rows < p->total_tokens))
    return MSA_ERR_SHAPE;
  if (!(p->softmax_scale > 0.f)) return MSA_ERR_INVALID;
  if (p->dq_mode != MSA_DQ_RECOMPUTE && p->dq_mode != MSA_DQ_ATOMIC_POOL &&
      p->dq_mode != MSA_DQ_DS_BUFFER && p->dq_mode != MSA_DQ_ATOMIC_POOL_BF16)
    return MSA_ERR_INVALID;
  return MSA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

}  // namespace

extern "C" {

int msa_device_check(int device, int32_t* num_cus) {
  if (device < 0 || device >= kMaxDevices) return MSA_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_dev_state[device] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MSA_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_state[device] = ok ? 1 : 2;
    g_dev_cus[device] = prop.multiProcessorCount;
  }
  if (num_cus) *num_cus = g_dev_cus[device];
  return g_dev_state[device] == 1 ? MSA_OK : MSA_ERR_UNSUPPORTED;
}

int msa_schedule_layout_of(const msa_problem* p, msa_schedule_layout* out) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!out) return MSA_ERR_INVALID;
  *out = msa::schedule_layout(*p);
  return MSA_OK;
}

int msa_build_schedule_kv(const msa_problem* p, const int32_t* cu_seqlens, const int32_t* sel,
                          const int32_t* kv_starts, int32_t* sched, void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!cu_seqlens || !sched || (!sel && p->num_chunks > 0)) return MSA_ERR_INVALID;
  if (!aligned16(sched)) return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(
      msa::launch_build_schedule(*p, cu_seqlens, sel, kv_starts, sched, L, (hipStream_t)stream));
}

int msa_build_schedule(const msa_problem* p, const int32_t* cu_seqlens, const int32_t* sel,
                       int32_t* sched, void* stream) {
  return msa_build_schedule_kv(p, cu_seqlens, sel, nullptr, sched, stream);
}

int msa_forward(const msa_problem* p, const void* q, const void* k, const void* v,
                const int32_t* cu_seqlens, const int32_t* sched, void* out, float* lse, void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!cu_seqlens || !sched || (p->total_tokens > 0 && (!q || !k || !v || !out || !lse)))
    return MSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(sched))
    return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(
      msa::launch_forward(*p, q, k, v, cu_seqlens, sched, L, out, lse, (hipStream_t)stream));
}

int msa_forward_kv_scratch_bytes(const msa_problem* p, size_t* bytes) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->block_size != 64) return MSA_ERR_UNSUPPORTED;
  if (!bytes) return MSA_ERR_INVALID;
  *bytes = msa::forward_kv_scratch_layout(*p).total;
  return MSA_OK;
}

int msa_forward_kv(const msa_problem* p, const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens, const int32_t* sched, void* scratch, void* out, float* lse,
                   void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->block_size != 64) return MSA_ERR_UNSUPPORTED;
  if (!cu_seqlens || !sched || (p->total_tokens > 0 && (!q || !k || !v || !out || !lse || !scratch)))
    return MSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(sched) ||
      !aligned16(scratch) || !aligned16(lse))
    return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(
      msa::launch_forward_kv(*p, q, k, v, cu_seqlens, sched, L, scratch, out, lse, (hipStream_t)stream));
}

int msa_backward_scratch_bytes(const msa_problem* p, size_t* bytes) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_INVALID;
  *bytes = msa::backward_scratch_layout(*p).total;
  return MSA_OK;
}

int msa_backward_preprocess(const msa_problem* p, const void* out, const void* dout, void* scratch,
                            void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (p->total_tokens > 0 && (!out || !dout || !scratch)) return MSA_ERR_INVALID;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(scratch)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_backward_preprocess(*p, out, dout, scratch, (hipStream_t)stream));
}

int msa_backward_main(const msa_problem* p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, const int32_t* cu_seqlens,
                      const int32_t* sched, void* scratch, void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!cu_seqlens || !sched || (p->total_tokens > 0 && (!q || !k || !v || !dout || !lse || !scratch)))
    return MSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(scratch) || !aligned16(sched))
    return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(msa::launch_backward_main(*p, q, k, v, dout, lse, cu_seqlens, sched, L, scratch,
                                              (hipStream_t)stream));
}

int msa_backward_dq(const msa_problem* p, const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, const int32_t* cu_seqlens,
                    const int32_t* sched, const void* scratch, void* dq, void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!cu_seqlens || !sched ||
      (p->total_tokens > 0 && (!q || !k || !v || !dout || !lse || !scratch || !dq)))
    return MSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(scratch) ||
      !aligned16(sched) || !aligned16(dq))
    return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(msa::launch_backward_dq(*p, q, k, v, dout, lse, cu_seqlens, sched, L, scratch, dq,
                                            (hipStream_t)stream));
}

int msa_backward_postprocess(const msa_problem* p, const int32_t* sched, const void* scratch, void* dq,
                             void* dk, void* dv, void* stream) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  if (!sched || (p->total_tokens > 0 && (!scratch || !dq || !dk || !dv))) return MSA_ERR_INVALID;
  if (!aligned16(scratch) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(sched))
    return MSA_ERR_ALIGN;
  const msa_schedule_layout L = msa::schedule_layout(*p);
  return hip_status(msa::launch_backward_postprocess(*p, sched, L, scratch, dq, dk, dv, (hipStream_t)stream));
}

int msa_backward(const msa_problem* p, const void* q, const void* k, const void* v, const void* out,
                 const void* dout, const float* lse, const int32_t* cu_seqlens, const int32_t* sched,
                 void* scratch, void* dq, void* dk, void* dv, void* stream) {
  int st = msa_backward_preprocess(p, out, dout, scratch, stream);
  if (st != MSA_OK) return st;
  st = msa_backward_main(p, q, k, v, dout, lse, cu_seqlens, sched, scratch, stream);
  if (st != MSA_OK) return st;
  st = msa_backward_dq(p, q, k, v, dout, lse, cu_seqlens, sched, scratch, dq, stream);
  if (st != MSA_OK) return st;
  return msa_backward_postprocess(p, sched, scratch, dq, dk, dv, stream);
}

static int check_index_problem(const msa_problem* p) {
  const int st = check_problem(p);
  if (st != MSA_OK) return st;
  const int64_t max_doc_blocks = ((int64_t)p->max_doc_chunks * 8 + p->block_size - 1) / p->block_size;
  if (max_doc_blocks > MSA_INDEX_MAX_DOC_BLOCKS) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_kv_heads * (p->num_chunks + p->num_kblocks) > INT32_MAX) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int msa_index_scratch_bytes(const msa_problem* p, size_t* bytes) {
  const int st = check_index_problem(p);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_INVALID;
  *bytes = msa::index_scratch_layout(*p).total;
  return MSA_OK;
}

int msa_index_select(const msa_problem* p, const void* qi, const void* ki, const int32_t* cu_seqlens,
                     void* scratch, int32_t* sel, void* stream) {
  const int st = check_index_problem(p);
  if (st != MSA_OK) return st;
  if (!cu_seqlens || !scratch || (p->num_chunks > 0 && !sel) || (p->total_tokens > 0 && (!qi || !ki)))
    return MSA_ERR_INVALID;
  if (!aligned16(qi) || !aligned16(ki) || !aligned16(scratch) || ((uintptr_t)sel & 3u) != 0)
    return MSA_ERR_ALIGN;
  return hip_status(msa::launch_index_select(*p, qi, ki, cu_seqlens, scratch, sel, (hipStream_t)stream));
}

int64_t msa_grid_launch_bound(int64_t capacity, int32_t num_cus) {
  if (capacity < 0 || num_cus < 1) return -1;
  return msa::grid_launch_bound(capacity, num_cus);
}

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID: return "invalid argument (null pointer or bad size)";
    case MSA_ERR_UNSUPPORTED: return "unsupported device or problem size";
    case MSA_ERR_SHAPE: return "inconsistent sizes";
    case MSA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case MSA_ERR_HIP: return "HIP runtime error";
    case MSA_ERR_SCRATCH_LIMIT:
      return "problem needs more scratch than the static buffer of msa_backward_noalloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"
