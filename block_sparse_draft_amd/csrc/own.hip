// Own-block mask: a draft block also attends to its own draft tokens, whose
// keys and values are a query-sized segment held with the queries.  Under
// Split-KV that segment is one more partial per row, merged exactly with the
// context chunks' partials (pages: Split-KV article, "Split-KV's Core
// Mechanism").  The work is tiny next to the context chunks (block keys per
// row instead of thousands), so these kernels stage the block's keys in LDS
// and compute in fp32 on the vector ALUs.
//
// One workgroup per (draft block, KV head): its G*B rows (the G query heads of
// the KV head times the block's B tokens) against the block's B own keys.
// Four lanes share a row, each holding a quarter of the head dimension.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int OWN_THREADS = 256;
constexpr int OWN_RG = 32;                               // rows per LDS group of the own-block dK/dV pass
constexpr int OWN_TASKS = 64 * (128 / 8) / OWN_THREADS;  // (own key, 8 columns) tasks per thread at block 64
// The host limits block <= 64 and G*B*B <= 8192, so the dynamic LDS of these
// kernels stays within 2*64*128*4 + 2*8192*4 + 2*32*128*2 bytes = 144 KB.

__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

// N consecutive elements (16-byte aligned) widened to fp32, in 16-byte loads.
template <int N>
__device__ __forceinline__ void ld_row(const float* p, float* out) {
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * k);
    out[4 * k] = v[0]; out[4 * k + 1] = v[1]; out[4 * k + 2] = v[2]; out[4 * k + 3] = v[3];
  }
}
template <int N>
__device__ __forceinline__ void ld_row(const uint16_t* p, float* out) {
#pragma unroll
  for (int k = 0; k < N / 8; ++k) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      out[8 * k + 2 * u] = __uint_as_float(w[u] << 16);
      out[8 * k + 2 * u + 1] = __uint_as_float(w[u] & 0xffff0000u);
    }
  }
}

// 8 consecutive elements (16-byte aligned for bf16, 32 for fp32) widened to fp32.
__device__ __forceinline__ void ld_chunk8(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
  out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
}
__device__ __forceinline__ void ld_chunk8(const uint16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    out[2 * u] = __uint_as_float(w[u] << 16);
    out[2 * u + 1] = __uint_as_float(w[u] & 0xffff0000u);
  }
}

// Sequence of token t: q_off[s] <= t < q_off[s + 1].
__device__ __forceinline__ int seq_of(const int64_t* q_off, int n_seq, int64_t t) {
  int lo = 0, hi = n_seq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q_off[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Sum of a quad of lanes (the four lanes of one row).
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// ---------------------------------------------------------------------------
// forward: the own-block partial of every row
// ---------------------------------------------------------------------------

// Dynamic LDS of the own-block kernels: K and V of the block's B own keys as
// fp32 [B][D] each (the backward adds P and dS, fp32 [G*B][B] each).
extern __shared__ float own_lds[];

template <typename T, int D>
__global__ __launch_bounds__(OWN_THREADS) void own_fwd_kernel(OwnFwdArgs a) {
  float (*sK)[D] = reinterpret_cast<float (*)[D]>(own_lds);
  float (*sV)[D] = reinterpret_cast<float (*)[D]>(own_lds + a.block * D);
  __shared__ unsigned long long s_base;
  constexpr int D4 = D / 4;
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int B = a.block, G = a.group;
  const int64_t t0 = (int64_t)blockIdx.x * B;  // first draft token of the block
  const int s = seq_of(a.q_off, a.n_seq, t0);
  const int64_t q0 = a.q_off[s], mq = a.q_off[s + 1] - q0;
  const int64_t n_ctx = a.kv_off[s + 1] - a.kv_off[s];
  const int64_t n_chunk = (n_ctx + a.chunk - 1) / a.chunk;

  // first partial row of sequence s: every earlier sequence has its chunks and its own-block partial
  if (tid == 0) s_base = 0;
  __syncthreads();
  unsigned long long part = 0;
  for (int i = tid; i < s; i += OWN_THREADS) {
    const int64_t n = a.kv_off[i + 1] - a.kv_off[i];
    part += (unsigned long long)(((n + a.chunk - 1) / a.chunk + 1) * a.hq * (a.q_off[i + 1] - a.q_off[i]));
  }
  if (part) atomicAdd(&s_base, part);
  const T* Ko = static_cast<const T*>(a.k_own);
  const T* Vo = static_cast<const T*>(a.v_own);
  for (int idx = tid; idx < B * D; idx += OWN_THREADS) {
    const int j = idx / D, x = idx % D;
    const int64_t off = (t0 + j) * a.own_st + (int64_t)g * a.own_sh + x;
    sK[j][x] = ld_elem(Ko, off);
    sV[j][x] = ld_elem(Vo, off);
  }
  __syncthreads();
  const int64_t own_base = (int64_t)s_base + n_chunk * a.hq * mq;  // first row of the own-block partial

  // Four lanes per row; lane q4 holds the 8-element chunks q4, q4 + 4, ... of
  // the head dimension, so the four lanes of a row read and write contiguous
  // 16- and 32-byte pieces.  Online softmax in the exp2 domain.
  const T* Q = static_cast<const T*>(a.q);
  const int q4 = tid & 3;
  constexpr int NCH = D / 32;  // chunks per lane
  const float c2 = a.sm_scale * kLog2e;
  for (int r = tid >> 2; r < G * B; r += OWN_THREADS / 4) {
    const int hl = r / B, i = r % B;
    const int h = g * G + hl;
    const int64_t t = t0 + i;
    float qv[D4];
#pragma unroll
    for (int k = 0; k < NCH; ++k) ld_chunk8(Q + t * a.q_st + (int64_t)h * a.q_sh + (q4 + 4 * k) * 8, qv + 8 * k);
    float m2 = -INFINITY, l = 0.f, o[D4];
#pragma unroll
    for (int x = 0; x < D4; ++x) o[x] = 0.f;
    for (int j = 0; j < B; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qv[8 * k + e], sK[j][(q4 + 4 * k) * 8 + e], dot);
      const float sc2 = quad_sum(dot) * c2;  // log2 units
      const float mn2 = fmaxf(m2, sc2);
      const float alpha = fast_exp2(m2 - mn2);  // 0 while m2 is -inf
      const float p = fast_exp2(sc2 - mn2);
      l = l * alpha + p;
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[8 * k + e] = fmaf(p, sV[j][(q4 + 4 * k) * 8 + e], o[8 * k + e] * alpha);
      m2 = mn2;
    }
    const int64_t row = own_base + (int64_t)h * mq + (t - q0);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      float* op = a.o_part + row * D + (q4 + 4 * k) * 8;
      *reinterpret_cast<f32x4*>(op) = f32x4{o[8 * k], o[8 * k + 1], o[8 * k + 2], o[8 * k + 3]};
      *reinterpret_cast<f32x4*>(op + 4) = f32x4{o[8 * k + 4], o[8 * k + 5], o[8 * k + 6], o[8 * k + 7]};
    }
    if (q4 == 0) {
      a.m_part[row] = m2 * kLn2;
      a.lse_part[row] = (m2 + __log2f(l)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// backward: dK_own, dV_own and the own-block dQ partial
// ---------------------------------------------------------------------------

// Rows come from the backward's packed copies: the G*B rows of (block, KV
// head) are consecutive there.  P = exp2(s*log2e - LSE*log2e),
// dS = P (dO.v - Delta); the dQ partial (unscaled, like the chunks') goes to
// the sequence's partial index C_s, summed by the finalize kernel.
__global__ __launch_bounds__(OWN_THREADS) void own_bwd_kernel(BwdArgs a) {
  constexpr int D = 128, D4 = D / 4;
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int B = a.block, G = a.group, R = G * B;
  float (*sK)[D] = reinterpret_cast<float (*)[D]>(own_lds);
  float (*sV)[D] = reinterpret_cast<float (*)[D]>(own_lds + B * D);
  float* sP = own_lds + 2 * B * D;
  float* sDS = sP + R * B;
  const int64_t t0 = (int64_t)blockIdx.x * B;
  const int s = seq_of(a.q_off, a.n_seq, t0);
  const int64_t q0 = a.q_off[s], mq = a.q_off[s + 1] - q0;
  const int64_t n_ctx = a.kv_off[s + 1] - a.kv_off[s];
  const int64_t n_chunk = (n_ctx + a.chunk - 1) / a.chunk;
  const int64_t blk = (t0 - q0) / B;
  const int64_t P0 = q0 * a.hq + (int64_t)g * G * mq + blk * R;  // packed row of (block, KV head)
  const int64_t dq_base = a.part_base[s] + n_chunk * a.hq * mq;

  const uint16_t* Ko = static_cast<const uint16_t*>(a.k_own);
  const uint16_t* Vo = static_cast<const uint16_t*>(a.v_own);
  for (int idx = tid; idx < B * D; idx += OWN_THREADS) {
    const int j = idx / D, x = idx % D;
    const int64_t off = (t0 + j) * a.own_st + (int64_t)g * a.own_sh + x;
    sK[j][x] = bf16_bits_to_f32(Ko[off]);
    sV[j][x] = bf16_bits_to_f32(Vo[off]);
  }
  __syncthreads();

  // ---- P, dS of every (row, own key); the row's dQ partial.  Four lanes
  //      per row; lane q4 holds the 8-element chunks q4, q4 + 4, ... ----
  const int q4 = tid & 3;
  constexpr int NCH = D / 32;
  for (int r = tid >> 2; r < R; r += OWN_THREADS / 4) {
    const int64_t P = P0 + r;
    const int hl = r / B, i = r % B;
    const int h = g * G + hl;
    float qv[D4], dov[D4], dq[D4];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      ld_chunk8(a.qp + P * D + (q4 + 4 * k) * 8, qv + 8 * k);
      ld_chunk8(a.dop + P * D + (q4 + 4 * k) * 8, dov + 8 * k);
    }
#pragma unroll
    for (int x = 0; x < D4; ++x) dq[x] = 0.f;
    const float lse2 = a.lsep[P], del = a.deltap[P];
    for (int j = 0; j < B; ++j) {
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sd = fmaf(qv[8 * k + e], sK[j][(q4 + 4 * k) * 8 + e], sd);
          pd = fmaf(dov[8 * k + e], sV[j][(q4 + 4 * k) * 8 + e], pd);
        }
      sd = quad_sum(sd);
      pd = quad_sum(pd);
      const float p = fast_exp2(sd * a.scale_log2 - lse2);
      const float ds = p * (pd - del);
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) dq[8 * k + e] = fmaf(ds, sK[j][(q4 + 4 * k) * 8 + e], dq[8 * k + e]);
      if (q4 == 0) {
        sP[r * B + j] = p;
        sDS[r * B + j] = ds;
      }
    }
    float* out = a.dq_part + (dq_base + (int64_t)h * mq + (t0 - q0) + i) * D;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      float* op = out + (q4 + 4 * k) * 8;
      *reinterpret_cast<f32x4*>(op) = f32x4{dq[8 * k], dq[8 * k + 1], dq[8 * k + 2], dq[8 * k + 3]};
      *reinterpret_cast<f32x4*>(op + 4) = f32x4{dq[8 * k + 4], dq[8 * k + 5], dq[8 * k + 6], dq[8 * k + 7]};
    }
  }

  // ---- dK_own = scale * dS^T Q, dV_own = P^T dO over the block's rows ----
  // task = (own key j, 8 head-dim columns), at most OWN_TASKS per thread; the
  // packed Q and dO rows pass through LDS OWN_RG rows at a time, in row order.
  uint16_t* sQb = reinterpret_cast<uint16_t*>(sDS + R * B);
  uint16_t* sOb = sQb + OWN_RG * D;
  const int n_task = B * (D / 8);
  float ak[OWN_TASKS][8], av[OWN_TASKS][8];
#pragma unroll
  for (int u = 0; u < OWN_TASKS; ++u)
#pragma unroll
    for (int x = 0; x < 8; ++x) ak[u][x] = av[u][x] = 0.f;
  for (int r0 = 0; r0 < R; r0 += OWN_RG) {
    const int nr = min(OWN_RG, R - r0);
    __syncthreads();  // P, dS written (first group); the previous group's rows consumed
    for (int idx = tid; idx < nr * (D / 8); idx += OWN_THREADS) {
      const int rr = idx / (D / 8), c8 = idx % (D / 8);
      const int64_t off = (P0 + r0 + rr) * D + c8 * 8;
      *reinterpret_cast<uint4*>(sQb + rr * D + c8 * 8) = *reinterpret_cast<const uint4*>(a.qp + off);
      *reinterpret_cast<uint4*>(sOb + rr * D + c8 * 8) = *reinterpret_cast<const uint4*>(a.dop + off);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < OWN_TASKS; ++u) {
      const int task = tid + u * OWN_THREADS;
      if (task >= n_task) break;
      const int j = task / (D / 8), c8 = task % (D / 8);
      for (int rr = 0; rr < nr; ++rr) {
        const int r = r0 + rr;
        const float ds = sDS[r * B + j], p = sP[r * B + j];
        const uint4 qw = *reinterpret_cast<const uint4*>(sQb + rr * D + c8 * 8);
        const uint4 ow = *reinterpret_cast<const uint4*>(sOb + rr * D + c8 * 8);
        const uint32_t qa[4] = {qw.x, qw.y, qw.z, qw.w}, oa[4] = {ow.x, ow.y, ow.z, ow.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ak[u][2 * w] = fmaf(ds, __uint_as_float(qa[w] << 16), ak[u][2 * w]);
          ak[u][2 * w + 1] = fmaf(ds, __uint_as_float(qa[w] & 0xffff0000u), ak[u][2 * w + 1]);
          av[u][2 * w] = fmaf(p, __uint_as_float(oa[w] << 16), av[u][2 * w]);
          av[u][2 * w + 1] = fmaf(p, __uint_as_float(oa[w] & 0xffff0000u), av[u][2 * w + 1]);
        }
      }
    }
  }
  uint16_t* dKo = static_cast<uint16_t*>(a.dk_own);
  uint16_t* dVo = static_cast<uint16_t*>(a.dv_own);
#pragma unroll
  for (int u = 0; u < OWN_TASKS; ++u) {
    const int task = tid + u * OWN_THREADS;
    if (task >= n_task) break;
    const int j = task / (D / 8), c8 = task % (D / 8);
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      kw[w] = (uint32_t)f32_to_bf16_bits(a.sm_scale * ak[u][2 * w]) |
              ((uint32_t)f32_to_bf16_bits(a.sm_scale * ak[u][2 * w + 1]) << 16);
      vw[w] = (uint32_t)f32_to_bf16_bits(av[u][2 * w]) | ((uint32_t)f32_to_bf16_bits(av[u][2 * w + 1]) << 16);
    }
    const int64_t off = (t0 + j) * a.own_st + (int64_t)g * a.own_sh + c8 * 8;
    *reinterpret_cast<uint4*>(dKo + off) = uint4{kw[0], kw[1], kw[2], kw[3]};
    *reinterpret_cast<uint4*>(dVo + off) = uint4{vw[0], vw[1], vw[2], vw[3]};
  }
}

}  // namespace

hipError_t launch_own_fwd(const OwnFwdArgs& a, int dtype, int d, int64_t n_blocks, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  TimedLaunch t(kOwnFwd, stream);
  const dim3 grid((unsigned)n_blocks, (unsigned)a.hkv);
  const size_t lds = (size_t)2 * a.block * d * sizeof(float);
  if (dtype == SKV_BF16)
    hipLaunchKernelGGL((own_fwd_kernel<uint16_t, 128>), grid, dim3(OWN_THREADS), lds, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((own_fwd_kernel<float, 128>), grid, dim3(OWN_THREADS), lds, stream, a);
  else
    hipLaunchKernelGGL((own_fwd_kernel<float, 64>), grid, dim3(OWN_THREADS), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_own_bwd(const BwdArgs& a, int64_t n_blocks, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  TimedLaunch t(kOwnBwd, stream);
  const size_t lds = (size_t)(2 * a.block * 128 + 2 * a.group * a.block * a.block) * sizeof(float) +
                     (size_t)2 * OWN_RG * 128 * sizeof(uint16_t);
  hipLaunchKernelGGL(own_bwd_kernel, dim3((unsigned)n_blocks, (unsigned)a.hkv), dim3(OWN_THREADS), lds, stream, a);
  return hipGetLastError();
}

}  // namespace skv
