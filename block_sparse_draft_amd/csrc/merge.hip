// Exact log-sum-exp merge of Split-KV partials (pages: Split-KV article,
// "Split-KV's Core Mechanism": shard-local results are aggregated so that the
// result equals the unsharded one).  Bandwidth-bound: every visible partial
// row (d fp32) is read once, every output row written once.
//
// Workgroup = 32 consecutive query rows of one head.  Step A: one thread per
// row folds the n_part log-sum-exps into the merged LSE.  Then, 64 partials at
// a time, step B computes the weights exp(m_c - LSE) (0 for partials the row
// does not see) into LDS with row-coalesced loads, and step C accumulates the
// weighted partial rows, 16 bytes per lane, skipping zero-weight partials so
// their (unwritten) rows are never read.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int MROWS = 32;   // rows per workgroup
constexpr int CBLK = 64;    // partials per weight block

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;              // lanes per output row (4 floats each)
  constexpr int SLOTS = 256 / LPR;        // row slots per workgroup
  constexpr int RPS = MROWS / SLOTS;      // rows handled per slot
  __shared__ float sLse[MROWS];
  __shared__ float sW[CBLK][MROWS];

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * MROWS;
  const int64_t hm = (int64_t)h * a.mq;
  const int64_t pstride = (int64_t)a.hq * a.mq;  // rows between consecutive partials

  // ---- step A: merged LSE of each row ----
  if (tid < MROWS) {
    const int64_t r = r0 + tid;
    float lse = -INFINITY;
    if (r < a.mq) {
      float mx = -INFINITY, sum = 0.f;
      for (int c = 0; c < a.n_part; ++c) {
        const float x = a.lse_part[c * pstride + hm + r];
        if (x == -INFINITY) continue;
        if (x > mx) {
          sum = sum * expf(mx - x) + 1.f;
          mx = x;
        } else {
          sum += expf(x - mx);
        }
      }
      lse = mx == -INFINITY ? -INFINITY : mx + logf(sum);
      a.lse_out[r * a.lse_st + h] = lse;
    }
    sLse[tid] = lse;
  }

  const int slot = tid / LPR, ln = tid % LPR;
  f32x4 acc[RPS];
#pragma unroll
  for (int i = 0; i < RPS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int cb = 0; cb < a.n_part; cb += CBLK) {
    __syncthreads();
    // ---- step B: weights of partials [cb, cb + 64) for the 32 rows ----
    for (int idx = tid; idx < CBLK * MROWS; idx += 256) {
      const int rr = idx % MROWS, cc = idx / MROWS;
      const int c = cb + cc;
      const int64_t r = r0 + rr;
      float w = 0.f;
      if (c < a.n_part && r < a.mq) {
        const float lc = a.lse_part[c * pstride + hm + r];
        const float L = sLse[rr];
        if (lc != -INFINITY && L != -INFINITY) w = expf(a.m_part[c * pstride + hm + r] - L);
      }
      sW[cc][rr] = w;
    }
    __syncthreads();
    // ---- step C: accumulate weighted partial rows ----
    const int cn = min(CBLK, a.n_part - cb);
    for (int cc = 0; cc < cn; ++cc) {
      const float* base = a.o_part + ((int64_t)(cb + cc) * pstride + hm + r0) * D + ln * 4;
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
        const int rr = slot * RPS + i;
        const float w = sW[cc][rr];
        if (w != 0.f) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(base + (int64_t)rr * D);
          acc[i] += w * v;
        }
      }
    }
  }

  // ---- write O ----
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int rr = slot * RPS + i;
    const int64_t r = r0 + rr;
    if (r >= a.mq) continue;
    const int64_t off = r * a.o_st + (int64_t)h * a.o_sh + ln * 4;
    if (a.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(a.o_out) + off;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_bits(acc[i][0]) | ((uint32_t)f32_to_bf16_bits(acc[i][1]) << 16);
      pk.y = (uint32_t)f32_to_bf16_bits(acc[i][2]) | ((uint32_t)f32_to_bf16_bits(acc[i][3]) << 16);
      *reinterpret_cast<uint2*>(o) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.o_out) + off) = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t stream) {
  if (a.mq == 0) return hipSuccess;
  dim3 grid((unsigned)((a.mq + MROWS - 1) / MROWS), (unsigned)a.hq);
  TimedLaunch t(kMerge, stream);
  if (d == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
