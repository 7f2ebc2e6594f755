// Split-KV partial forward in fp32 (head_dim 64 or 128) on the vector ALU.
//
// Same contract as the bf16 MFMA kernel (pages: Split-KV article, "Split-KV's
// Core Mechanism": one query-sized partial per KV chunk, aggregated exactly
// later), written for accuracy rather than speed: one thread owns one packed
// query row of the item, keeps q and the unnormalised output in registers and
// walks the row's visible keys of the chunk one by one with an online softmax.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  const int GB = a.group * a.block;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int64_t slot_end = a.worker_off[blockIdx.x + 1];
  for (int64_t slot = a.worker_off[blockIdx.x]; slot < slot_end; ++slot) {
    const skv_item it = a.items[slot];
    const int s = it.seq;
    const int64_t q0 = a.q_off[s];
    const int64_t mq = a.q_off[s + 1] - q0;
    const int64_t k0 = a.kv_off[s];
    const int n_ctx = (int)(a.kv_off[s + 1] - k0);
    const int64_t blk0 = q0 / a.block;
    // keys of the item's chunks: [chunk*L, (chunk + n_chunk)*L) inside the context
    const int klo = it.chunk * a.chunk;
    const int khi = (int)min((int64_t)(it.chunk + max(1, it.n_chunk)) * a.chunk, (int64_t)n_ctx);
    const int nrows = (it.hi - it.lo) * GB;
    for (int p = threadIdx.x; p < nrows; p += blockDim.x) {
      const int b = it.lo + p / GB;
      const int hl = (p / a.block) % a.group;
      const int i = p % a.block;
      const int e = min(a.anchor[blk0 + b] + a.end_shift, n_ctx);
      const int vend = min(khi, e);
      const int h = it.kv_head * a.group + hl;
      const int64_t r = (int64_t)b * a.block + i;
      const int64_t prow = it.part_base + (int64_t)h * mq + r;
      if (vend <= klo) {
        a.m_part[prow] = -INFINITY;
        a.lse_part[prow] = -INFINITY;
        continue;
      }
      float q[D], o[D];
      const float* qp = Q + (q0 + r) * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
      for (int x = 0; x < D; ++x) { q[x] = qp[x]; o[x] = 0.f; }
      float m = -INFINITY, l = 0.f;
      for (int j = klo; j < vend; ++j) {
        const float* kp = K + (k0 + j) * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
        const float* vp = V + (k0 + j) * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(q[x], kp[x], dot);
        const float sx = dot * a.scale_log2;
        const float m_new = fmaxf(m, sx);
        const float alpha = exp2f(m - m_new);
        const float pj = exp2f(sx - m_new);
        l = l * alpha + pj;
#pragma unroll
        for (int x = 0; x < D; ++x) o[x] = fmaf(pj, vp[x], o[x] * alpha);
        m = m_new;
      }
      a.m_part[prow] = m * kLn2;
      a.lse_part[prow] = (m + log2f(l)) * kLn2;
      float* op = a.o_part + prow * D;
#pragma unroll
      for (int x = 0; x < D; ++x) op[x] = o[x];
    }
  }
  record_ticks(a.ticks, blockIdx.x, t_start);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, int n_workers, hipStream_t stream) {
  TimedLaunch t(kFwdF32, stream);
  if (d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(n_workers), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(n_workers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
