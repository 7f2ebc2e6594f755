// Exact log-sum-exp merge of Split-KV partials (pages: Split-KV article,
// "Split-KV's Core Mechanism": shard-local results are aggregated so that the
// result equals the unsharded one).  Bandwidth-bound: every visible partial
// row (d fp32) is read once, every output row written once.
//
// Workgroup = 32 consecutive query rows of one head.  Step A: eight lanes
// per row fold the n_part log-sum-exps (each lane a strided eighth, then the
// eight partial folds combined) into the merged LSE.  Then, 64 partials at a
// time, step B lists per row the partials with a nonzero weight
// exp(m_c - LSE) in ascending partial order (0 for partials the row does not
// see, whose unwritten rows are never read), and step C accumulates the
// weighted partial rows of each list, 16 bytes per lane, four independent
// loads at a time.  The order of every sum is fixed: bitwise deterministic.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int MROWS = 32;   // rows per workgroup
constexpr int CBLK = 64;    // partials per weight block
constexpr int LPRA = 8;     // lanes per row in steps A and B

// (max, sum of exp(x - max)) of two disjoint sets combined.
__device__ __forceinline__ void lse_combine(float& mx, float& sum, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (mx == -INFINITY) { mx = m2; sum = s2; return; }
  const float m = fmaxf(mx, m2);
  sum = sum * expf(mx - m) + s2 * expf(m2 - m);
  mx = m;
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;              // lanes per output row (4 floats each)
  constexpr int SLOTS = 256 / LPR;        // row slots per workgroup
  constexpr int RPS = MROWS / SLOTS;      // rows handled per slot
  __shared__ float sLse[MROWS];
  __shared__ float sW[MROWS][CBLK];       // nonzero weights of the block, per row, ascending partial
  __shared__ int sC[MROWS][CBLK];         // their partial index
  __shared__ int sN[MROWS];
  __shared__ int64_t sBase[MROWS];        // first partial row of each row, and the partial stride
  __shared__ int64_t sStride[MROWS];
  __shared__ int sNp[MROWS];              // partials of each row's sequence
  __shared__ int sMaxNp;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * MROWS;

  // ---- each row's partial layout (its sequence, when rows of several sequences are merged) ----
  if (tid < 64) {
    int np = -1;
    if (tid < MROWS && r0 + tid < a.mq) {
      const int64_t t = r0 + tid;
      if (a.n_seq == 0) {
        sBase[tid] = (int64_t)h * a.mq + t;
        sStride[tid] = (int64_t)a.hq * a.mq;
        np = a.n_part;
      } else {
        int lo = 0, hi = a.n_seq;  // sequence of row t: q_off[lo] <= t < q_off[lo + 1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (a.q_off[mid] <= t) lo = mid; else hi = mid;
        }
        const int64_t q0 = a.q_off[lo], mqs = a.q_off[lo + 1] - q0;
        const int64_t stride = (int64_t)a.hq * mqs;
        sBase[tid] = a.part_base[lo] + (int64_t)h * mqs + (t - q0);
        sStride[tid] = stride;
        np = (int)((a.part_base[lo + 1] - a.part_base[lo]) / stride);
      }
    }
    if (tid < MROWS) sNp[tid] = np < 0 ? 0 : np;
    const int mx = wave_max_i(np);
    if (tid == 0) sMaxNp = mx < 0 ? 0 : mx;
  }
  __syncthreads();
  const int max_np = sMaxNp;
  const int ra = tid / LPRA, pa = tid % LPRA;    // steps A, B: row, lane within the row
  const int64_t rowa = r0 + ra;
  const bool live_a = rowa < a.mq;
  const int64_t base_a = sBase[ra], stride_a = sStride[ra];
  const int np_a = sNp[ra];

  // ---- step A: merged LSE of each row ----
  {
    float mx = -INFINITY, sum = 0.f;
    if (live_a) {
      for (int c0 = pa; c0 < np_a; c0 += 4 * LPRA) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * LPRA;
          x[u] = c < np_a ? a.lse_part[base_a + c * stride_a] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) lse_combine(mx, sum, x[u], 1.f);
      }
    }
#pragma unroll
    for (int o = 1; o < LPRA; o <<= 1) {
      const float m2 = __shfl_xor(mx, o), s2 = __shfl_xor(sum, o);
      lse_combine(mx, sum, m2, s2);
    }
    const float lse = mx == -INFINITY ? -INFINITY : mx + logf(sum);
    if (pa == 0) {
      if (live_a) a.lse_out[rowa * a.lse_st + h] = lse;
      sLse[ra] = lse;
    }
  }

  const int slot = tid / LPR, ln = tid % LPR;
  f32x4 acc[RPS];
#pragma unroll
  for (int i = 0; i < RPS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int cb = 0; cb < max_np; cb += CBLK) {
    __syncthreads();  // sLse written; the previous block's lists are consumed
    // ---- step B: this row's nonzero weights among partials [cb, cb + 64) ----
    {
      const float L = sLse[ra];
      int count = 0;
#pragma unroll
      for (int u = 0; u < CBLK / LPRA; ++u) {
        const int c = cb + u * LPRA + pa;
        float w = 0.f;
        if (live_a && c < np_a && L != -INFINITY) {
          const float lc = a.lse_part[base_a + c * stride_a];
          if (lc != -INFINITY) w = expf(a.m_part[base_a + c * stride_a] - L);
        }
        const uint64_t bal = __ballot(w != 0.f);
        const uint32_t bits = (uint32_t)(bal >> (lane & ~(LPRA - 1))) & ((1u << LPRA) - 1);
        if (w != 0.f) {
          const int pos = count + __popc(bits & ((1u << pa) - 1));
          sW[ra][pos] = w;
          sC[ra][pos] = c;
        }
        count += __popc(bits);
      }
      if (pa == 0) sN[ra] = count;
    }
    __syncthreads();
    // ---- step C: accumulate the listed partial rows ----
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
      const int rr = slot * RPS + i;
      const int n = sN[rr];
      const float* base = a.o_part + sBase[rr] * D + ln * 4;
      const int64_t pstride = sStride[rr] * D;
      int k = 0;
      for (; k + 4 <= n; k += 4) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4*>(base + (int64_t)sC[rr][k + u] * pstride);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[i] += sW[rr][k + u] * v[u];
      }
      for (; k < n; ++k) acc[i] += sW[rr][k] * *reinterpret_cast<const f32x4*>(base + (int64_t)sC[rr][k] * pstride);
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
