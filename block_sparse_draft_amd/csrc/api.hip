// Device entry points of libsplitkv: argument checks (host copies only, before
// any HIP call), then kernel launches on the caller's stream.
#include <cmath>
#include <mutex>

#include "internal.h"
#include "launch.h"

using namespace skv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_plan(const skv_plan* plan, int32_t kind) {
  if (!plan) return fail(SKV_EINVAL, "plan is NULL");
  if (plan->kind != kind) return fail(SKV_EPLAN, "plan kind %d does not match this call (%d)", plan->kind, kind);
  if (plan->n_workers < 1) return fail(SKV_EPLAN, "plan has %d workers", plan->n_workers);
  if (plan->n_items < 0 || plan->n_items > INT32_MAX)
    return fail(SKV_EPLAN, "plan item count %lld outside [0, 2^31)", (long long)plan->n_items);
  if (!plan->d_worker_off || !plan->d_claim || (plan->n_items > 0 && !plan->d_items))
    return fail(SKV_EPLAN, "plan arrays are NULL");
  if (plan->flags & ~SKV_PLAN_NO_STEAL) return fail(SKV_EPLAN, "unknown plan flags 0x%x", plan->flags);
  return SKV_OK;
}

int check_device_problem(const skv_problem* p) {
  // the anchor array is empty (and may be NULL) when the batch has no draft blocks
  if (!p->d_q_off || !p->d_kv_off || (!p->d_anchor && p->h_q_off[p->n_seq] > 0))
    return fail(SKV_EINVAL, "device offset/anchor arrays are NULL");
  return SKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SKV_EHIP, "%s: %s", what, hipGetErrorString(e));
  clear_error();
  return SKV_OK;
}

}  // namespace

extern "C" int sparse_attn_partial_fwd(const skv_problem* p, const skv_plan* plan, const void* q, const void* k,
                                       const void* v, float* o_part, float* m_part, float* lse_part, void* stream) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  if ((rc = check_device_problem(p))) return rc;
  if ((rc = check_plan(plan, SKV_ITEM_FWD))) return rc;
  // query-sized buffers may be NULL without query rows, K/V without context rows
  const int64_t tq = p->h_q_off[p->n_seq], tk = p->h_kv_off[p->n_seq];
  if ((tq && (!q || !o_part || !m_part || !lse_part)) || (tk && (!k || !v)))
    return fail(SKV_EINVAL, "tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part))
    return fail(SKV_ESHAPE, "q, k, v and o_part must be 16-byte aligned");
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.q_st = p->q_stride_tok; a.q_sh = p->q_stride_head;
  a.kv_st = p->kv_stride_tok; a.kv_sh = p->kv_stride_head;
  a.q_off = p->d_q_off; a.kv_off = p->d_kv_off; a.anchor = p->d_anchor;
  a.items = plan->d_items; a.worker_off = plan->d_worker_off; a.claim = plan->d_claim;
  a.ticks = plan->d_ticks; a.steal = !(plan->flags & SKV_PLAN_NO_STEAL);
  a.o_part = o_part; a.m_part = m_part; a.lse_part = lse_part;
  a.block = p->block; a.group = p->hq / p->hkv; a.hq = p->hq; a.chunk = p->chunk;
  a.fd_block = FastDiv::make(a.block); a.fd_group = FastDiv::make(a.group); a.fd_gb = FastDiv::make(a.block * a.group);
  a.end_shift = end_shift(p);
  a.sm_scale = p->sm_scale;
  a.scale_log2 = p->sm_scale * kLog2e_host;
  int64_t part_rows = 0;
  for (int s = 0; s < p->n_seq; ++s) {
    const SeqView v = seq_view(p, s);
    part_rows += n_partials(p, v.n) * p->hq * v.mq;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_neg_inf(m_part, lse_part, part_rows, plan->d_claim, plan->n_workers + 1, st);
  if (e != hipSuccess) return hip_status(e, "sparse_attn_partial_fwd launch");
  e = p->dtype == SKV_BF16 ? launch_fwd_bf16(a, plan->n_workers, st)
                                      : launch_fwd_f32(a, p->d, plan->n_workers, st);
  return hip_status(e, "sparse_attn_partial_fwd launch");
}

// Own-block limits: the own keys and values of a block, and the P / dS tile of
// its rows against them, are staged in LDS.
static int check_own_shape(const skv_problem* p) {
  if (p->mask != SKV_MASK_OWN_BLOCK) return fail(SKV_EINVAL, "the problem does not use the own-block mask");
  if (p->block > 64) return fail(SKV_ESHAPE, "own-block mask: block = %d > 64", p->block);
  if ((int64_t)(p->hq / p->hkv) * p->block * p->block > 8192)
    return fail(SKV_ESHAPE, "own-block mask: (hq/hkv) * block^2 = %lld > 8192",
                (long long)(p->hq / p->hkv) * p->block * p->block);
  return SKV_OK;
}

static int check_own_strides(const skv_problem* p, int64_t st, int64_t sh) {
  const int64_t vec = p->dtype == SKV_BF16 ? 8 : 4;
  if (sh < p->d || st < (int64_t)p->hkv * sh || st % vec || sh % vec)
    return fail(SKV_ESHAPE, "own-block strides (%lld, %lld) must be 16-byte multiples with tok >= hkv*head >= hkv*d",
                (long long)st, (long long)sh);
  return SKV_OK;
}

extern "C" int sparse_attn_own_fwd(const skv_problem* p, const void* q, const void* k_own, const void* v_own,
                                   int64_t own_stride_tok, int64_t own_stride_head, float* o_part, float* m_part,
                                   float* lse_part, void* stream) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  if ((rc = check_device_problem(p))) return rc;
  if ((rc = check_own_shape(p))) return rc;
  if ((rc = check_own_strides(p, own_stride_tok, own_stride_head))) return rc;
  if (p->h_q_off[p->n_seq] && (!q || !k_own || !v_own || !o_part || !m_part || !lse_part))
    return fail(SKV_EINVAL, "tensor pointer is NULL");  // all query-sized: NULL only without query rows
  if (!aligned16(q) || !aligned16(k_own) || !aligned16(v_own) || !aligned16(o_part))
    return fail(SKV_ESHAPE, "q, k_own, v_own and o_part must be 16-byte aligned");
  OwnFwdArgs a{};
  a.q = q; a.k_own = k_own; a.v_own = v_own;
  a.q_st = p->q_stride_tok; a.q_sh = p->q_stride_head; a.own_st = own_stride_tok; a.own_sh = own_stride_head;
  a.q_off = p->d_q_off; a.kv_off = p->d_kv_off;
  a.o_part = o_part; a.m_part = m_part; a.lse_part = lse_part;
  a.n_seq = p->n_seq; a.block = p->block; a.group = p->hq / p->hkv; a.hq = p->hq; a.hkv = p->hkv;
  a.chunk = p->chunk; a.sm_scale = p->sm_scale;
  const int64_t n_blocks = p->h_q_off[p->n_seq] / p->block;
  return hip_status(launch_own_fwd(a, p->dtype, p->d, n_blocks, static_cast<hipStream_t>(stream)),
                    "sparse_attn_own_fwd launch");
}

extern "C" int lse_merge(int32_t n_part, int32_t hq, int64_t mq, int32_t d, const float* o_part, const float* m_part,
                         const float* lse_part, void* o_out, int64_t o_stride_tok, int64_t o_stride_head,
                         int32_t out_dtype, float* lse_out, int64_t lse_stride_tok, void* stream) {
  if (n_part < 0 || hq < 1 || mq < 0) return fail(SKV_EINVAL, "bad counts n_part=%d hq=%d mq=%lld", n_part, hq,
                                                  (long long)mq);
  if (d != 64 && d != 128) return fail(SKV_ESHAPE, "lse_merge supports head_dim 64 or 128, got %d", d);
  if (out_dtype != SKV_F32 && out_dtype != SKV_BF16) return fail(SKV_EDTYPE, "unknown out_dtype %d", out_dtype);
  if (mq == 0) { clear_error(); return SKV_OK; }
  if (!o_out || !lse_out || (n_part > 0 && (!o_part || !m_part || !lse_part)))
    return fail(SKV_EINVAL, "tensor pointer is NULL");
  const int64_t vec = 4;  // 4 elements per lane store
  if (o_stride_tok < 1 || o_stride_head < d || lse_stride_tok < hq) return fail(SKV_ESHAPE, "bad output strides");
  if (o_stride_tok % vec || o_stride_head % vec) return fail(SKV_ESHAPE, "output strides must be multiples of 4");
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(o_out) & 7u))
    return fail(SKV_ESHAPE, "o_part must be 16-byte and o_out 8-byte aligned");
  if (mq > (int64_t)INT32_MAX * 32) return fail(SKV_ESHAPE, "mq too large");
  MergeArgs a{};
  a.o_part = o_part; a.m_part = m_part; a.lse_part = lse_part;
  a.o_out = o_out; a.lse_out = lse_out;
  a.mq = mq; a.o_st = o_stride_tok; a.o_sh = o_stride_head; a.lse_st = lse_stride_tok;
  a.n_part = n_part; a.hq = hq; a.out_bf16 = out_dtype == SKV_BF16;
  return hip_status(launch_merge(a, d, static_cast<hipStream_t>(stream)), "lse_merge launch");
}

extern "C" int lse_merge_all(const skv_problem* p, const int64_t* d_part_base, const float* o_part,
                             const float* m_part, const float* lse_part, void* o_out, float* lse_out,
                             void* stream) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  if ((rc = check_device_problem(p))) return rc;
  const int64_t rows = p->h_q_off[p->n_seq];
  if (rows == 0) { clear_error(); return SKV_OK; }
  if (!d_part_base || !o_part || !m_part || !lse_part || !o_out || !lse_out)
    return fail(SKV_EINVAL, "tensor pointer is NULL");
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(o_out) & 7u))
    return fail(SKV_ESHAPE, "o_part must be 16-byte and o_out 8-byte aligned");
  if (rows > (int64_t)INT32_MAX * 32) return fail(SKV_ESHAPE, "too many rows");
  MergeArgs a{};
  a.o_part = o_part; a.m_part = m_part; a.lse_part = lse_part;
  a.o_out = o_out; a.lse_out = lse_out;
  a.mq = rows; a.o_st = p->q_stride_tok; a.o_sh = p->q_stride_head; a.lse_st = p->hq;
  a.hq = p->hq; a.out_bf16 = p->dtype == SKV_BF16;
  a.q_off = p->d_q_off; a.part_base = d_part_base; a.n_seq = p->n_seq;
  return hip_status(launch_merge(a, p->d, static_cast<hipStream_t>(stream)), "lse_merge_all launch");
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of sparse_attn_bwd: dQ partials (the forward's partial layout);
// Q, dO, LSE (log2 units), Delta and the prefix end e_b copied into packed row
// order (sequence, KV head, packed row p = (b*G + hl)*B + i), which is the
// order both backward kernels walk; the first partial row of each sequence.
struct BwdWorkspace {
  size_t dq_part, dq_run, qp, dop, lsep, deltap, endp, part_base, total;
};
static BwdWorkspace bwd_workspace(const skv_problem* p) {
  int64_t rows = 0;
  for (int s = 0; s < p->n_seq; ++s) {
    const SeqView v = seq_view(p, s);
    rows += n_partials(p, v.n) * p->hq * v.mq;
  }
  const size_t prow = (size_t)p->h_q_off[p->n_seq] * (size_t)p->hq;  // packed rows
  BwdWorkspace w;
  w.dq_part = 0;
  w.dq_run = align256((size_t)rows * (size_t)p->d * sizeof(float));
  w.qp = w.dq_run + align256((size_t)rows * sizeof(int32_t));
  w.dop = w.qp + align256(prow * (size_t)p->d * 2);
  w.lsep = w.dop + align256(prow * (size_t)p->d * 2);
  w.deltap = w.lsep + align256(prow * sizeof(float));
  w.endp = w.deltap + align256(prow * sizeof(float));
  w.part_base = w.endp + align256(prow * sizeof(int32_t));
  w.total = w.part_base + align256((size_t)(p->n_seq + 1) * sizeof(int64_t));
  return w;
}

extern "C" size_t skv_bwd_workspace_bytes(const skv_problem* p) {
  if (skv_check_problem(p)) return 0;
  return bwd_workspace(p).total;
}

// Arguments of sparse_attn_bwd other than the workspace; SKV_OK if usable.
static int check_bwd_args(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                          const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, const skv_own_block* own) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  if (p->dtype != SKV_BF16) return fail(SKV_EDTYPE, "sparse_attn_bwd supports bf16 only");
  if ((rc = check_device_problem(p))) return rc;
  if ((rc = check_plan(plan_kv, SKV_ITEM_BWD))) return rc;
  if ((rc = check_plan(plan_q, SKV_ITEM_FWD))) return rc;
  if (plan_kv->d_claim == plan_q->d_claim) return fail(SKV_EPLAN, "the two plans must not share claim cursors");
  if (plan_kv->d_ticks && plan_kv->d_ticks == plan_q->d_ticks)
    return fail(SKV_EPLAN, "the two plans must not share a ticks array");
  // query-sized buffers may be NULL without query rows, K/V-sized ones without context rows
  const int64_t tq = p->h_q_off[p->n_seq], tk = p->h_kv_off[p->n_seq];
  if ((tq && (!q || !o || !lse || !dout || !dq)) || (tk && (!k || !v || !dk || !dv)))
    return fail(SKV_EINVAL, "tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(SKV_ESHAPE, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (p->mask == SKV_MASK_OWN_BLOCK) {
    if ((rc = check_own_shape(p))) return rc;
    if (!own || (tq && (!own->k || !own->v || !own->dk || !own->dv)))
      return fail(SKV_EINVAL, "the own-block mask needs own-block keys, values and gradient outputs");
    if ((rc = check_own_strides(p, own->stride_tok, own->stride_head))) return rc;
    if (!aligned16(own->k) || !aligned16(own->v) || !aligned16(own->dk) || !aligned16(own->dv))
      return fail(SKV_ESHAPE, "own-block tensors must be 16-byte aligned");
  } else if (own) {
    return fail(SKV_EINVAL, "own-block tensors given for the prefix mask");
  }
  return SKV_OK;
}

// The backward's launches with a validated workspace of bwd_workspace(p).total bytes.
static int launch_bwd(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                      const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                      void* dk, void* dv, void* workspace, const skv_own_block* own, void* stream);

extern "C" int sparse_attn_bwd(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                               const void* k, const void* v, const void* o, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                               const skv_own_block* own, void* stream) {
  int rc = check_bwd_args(p, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, own);
  if (rc) return rc;
  const BwdWorkspace ws = bwd_workspace(p);
  if (!workspace || workspace_bytes < ws.total)
    return fail(SKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(SKV_EWORKSPACE, "workspace must be 256-byte aligned");
  return launch_bwd(p, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, workspace, own, stream);
}

static int launch_bwd(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                      const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                      void* dk, void* dv, void* workspace, const skv_own_block* own, void* stream) {
  const BwdWorkspace ws = bwd_workspace(p);
  char* w = static_cast<char*>(workspace);
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.dq_part = reinterpret_cast<float*>(w + ws.dq_part);
  a.dq_run = reinterpret_cast<int32_t*>(w + ws.dq_run);
  a.qp = reinterpret_cast<uint16_t*>(w + ws.qp);
  a.dop = reinterpret_cast<uint16_t*>(w + ws.dop);
  a.lsep = reinterpret_cast<float*>(w + ws.lsep);
  a.deltap = reinterpret_cast<float*>(w + ws.deltap);
  a.endp = reinterpret_cast<int32_t*>(w + ws.endp);
  a.part_base = reinterpret_cast<int64_t*>(w + ws.part_base);
  a.q_st = p->q_stride_tok; a.q_sh = p->q_stride_head;
  a.kv_st = p->kv_stride_tok; a.kv_sh = p->kv_stride_head;
  a.q_off = p->d_q_off; a.kv_off = p->d_kv_off; a.anchor = p->d_anchor;
  a.kv_items = plan_kv->d_items; a.kv_worker_off = plan_kv->d_worker_off; a.kv_claim = plan_kv->d_claim;
  a.q_items = plan_q->d_items; a.q_worker_off = plan_q->d_worker_off; a.q_claim = plan_q->d_claim;
  a.kv_ticks = plan_kv->d_ticks; a.kv_steal = !(plan_kv->flags & SKV_PLAN_NO_STEAL);
  a.q_ticks = plan_q->d_ticks; a.q_steal = !(plan_q->flags & SKV_PLAN_NO_STEAL);
  a.total_q = p->h_q_off[p->n_seq];
  a.n_seq = p->n_seq; a.block = p->block; a.group = p->hq / p->hkv; a.hq = p->hq; a.hkv = p->hkv;
  a.chunk = p->chunk;
  a.end_shift = end_shift(p);
  a.own = p->mask == SKV_MASK_OWN_BLOCK;
  if (own) {
    a.k_own = own->k; a.v_own = own->v; a.dk_own = own->dk; a.dv_own = own->dv;
    a.own_st = own->stride_tok; a.own_sh = own->stride_head;
  }
  a.fd_block = FastDiv::make(a.block); a.fd_group = FastDiv::make(a.group); a.fd_gb = FastDiv::make(a.block * a.group);
  a.sm_scale = p->sm_scale; a.scale_log2 = p->sm_scale * kLog2e_host;
  hipStream_t st = static_cast<hipStream_t>(stream);
  a.kv_claim_n = plan_kv->n_workers + 1;  // cursors and the claimed-items count
  a.q_claim_n = plan_q->n_workers + 1;
  hipError_t e = launch_bwd_bf16(a, plan_kv->n_workers, plan_q->n_workers, st);
  return hip_status(e, "sparse_attn_bwd launch");
}

// ---------------------------------------------------------------------------
// sparse_attn_bwd without a caller workspace: the workspace lives in `scratch`,
// one copy per GPU, for callers that cannot allocate device memory.
// ---------------------------------------------------------------------------

// In host code `scratch` names a host-side stand-in, not the device array:
// only the address from hipGetSymbolAddress, taken once per device with that
// device current, is ever handed to kernels.
static __device__ __align__(256) char scratch[SKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

// Device address of `scratch` on the current device.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SKV_EHIP, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SKV_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

extern "C" int sparse_attn_bwd_noalloc(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q,
                                       const void* q, const void* k, const void* v, const void* o, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, const skv_own_block* own,
                                       void* stream) {
  int rc = check_bwd_args(p, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, own);
  if (rc) return rc;
  const size_t need = bwd_workspace(p).total;
  if (need > (size_t)SKV_NOALLOC_SCRATCH_BYTES)
    return fail(SKV_EWORKSPACE, "the backward of this problem needs %zu bytes of workspace, more than the %d bytes "
                "of the library's static scratch; use sparse_attn_bwd with a caller workspace", need,
                (int)SKV_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if ((rc = scratch_address(&ptr))) return rc;
  return launch_bwd(p, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, ptr, own, stream);
}
