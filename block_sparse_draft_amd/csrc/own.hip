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
// The host limits block <= 64 and G*B*B <= 8192, so the dynamic LDS of these
// kernels stays within 2*64*128*4 + 2*8192*4 bytes = 128 KB.

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

  const T* Q = static_cast<const T*>(a.q);
  const int q4 = tid & 3;
  for (int r = tid >> 2; r < G * B; r += OWN_THREADS / 4) {
    const int hl = r / B, i = r % B;
    const int h = g * G + hl;
    const int64_t t = t0 + i;
    float qv[D4];
    ld_row<D4>(Q + t * a.q_st + (int64_t)h * a.q_sh + q4 * D4, qv);
    float m = -INFINITY, l = 0.f, o[D4];
#pragma unroll
    for (int x = 0; x < D4; ++x) o[x] = 0.f;
    for (int j = 0; j < B; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < D4; ++x) dot = fmaf(qv[x], sK[j][q4 * D4 + x], dot);
      const float sc = quad_sum(dot) * a.sm_scale;
      const float mn = fmaxf(m, sc);
      const float alpha = expf(m - mn);  // 0 while m is -inf
      const float p = expf(sc - mn);
      l = l * alpha + p;
#pragma unroll
      for (int x = 0; x < D4; ++x) o[x] = fmaf(p, sV[j][q4 * D4 + x], o[x] * alpha);
      m = mn;
    }
    const int64_t row = own_base + (int64_t)h * mq + (t - q0);
#pragma unroll
    for (int x = 0; x < D4; ++x) a.o_part[row * D + q4 * D4 + x] = o[x];
    if (q4 == 0) {
      a.m_part[row] = m;
      a.lse_part[row] = m + logf(l);
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

  // ---- P, dS of every (row, own key); the row's dQ partial ----
  const int q4 = tid & 3;
  for (int r = tid >> 2; r < R; r += OWN_THREADS / 4) {
    const int64_t P = P0 + r;
    const int hl = r / B, i = r % B;
    const int h = g * G + hl;
    float qv[D4], dov[D4], dq[D4];
    ld_row<D4>(a.qp + P * D + q4 * D4, qv);
    ld_row<D4>(a.dop + P * D + q4 * D4, dov);
#pragma unroll
    for (int x = 0; x < D4; ++x) dq[x] = 0.f;
    const float lse2 = a.lsep[P], del = a.deltap[P];
    for (int j = 0; j < B; ++j) {
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int x = 0; x < D4; ++x) {
        sd = fmaf(qv[x], sK[j][q4 * D4 + x], sd);
        pd = fmaf(dov[x], sV[j][q4 * D4 + x], pd);
      }
      sd = quad_sum(sd);
      pd = quad_sum(pd);
      const float p = exp2f(sd * a.scale_log2 - lse2);
      const float ds = p * (pd - del);
#pragma unroll
      for (int x = 0; x < D4; ++x) dq[x] = fmaf(ds, sK[j][q4 * D4 + x], dq[x]);
      if (q4 == 0) {
        sP[r * B + j] = p;
        sDS[r * B + j] = ds;
      }
    }
    float* out = a.dq_part + (dq_base + (int64_t)h * mq + (t0 - q0) + i) * D + q4 * D4;
#pragma unroll
    for (int x = 0; x < D4; ++x) out[x] = dq[x];
  }
  __syncthreads();

  // ---- dK_own = scale * dS^T Q, dV_own = P^T dO over the block's rows ----
  // task = (own key j, 8 head-dim columns)
  uint16_t* dKo = static_cast<uint16_t*>(a.dk_own);
  uint16_t* dVo = static_cast<uint16_t*>(a.dv_own);
  for (int task = tid; task < B * (D / 8); task += OWN_THREADS) {
    const int j = task / (D / 8), c8 = task % (D / 8);
    float ak[8], av[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) ak[x] = av[x] = 0.f;
    // rows four at a time (R = G*B is a multiple of 4 whenever B is; a
    // ragged tail is clamped to the last row with zero weights)
    for (int r0 = 0; r0 < R; r0 += 4) {
      uint4 qw[4], ow[4];
      float ds[4], p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = min(r0 + u, R - 1);
        const int64_t P = P0 + r;
        qw[u] = *reinterpret_cast<const uint4*>(a.qp + P * D + c8 * 8);
        ow[u] = *reinterpret_cast<const uint4*>(a.dop + P * D + c8 * 8);
        const bool in = r0 + u < R;
        ds[u] = in ? sDS[r * B + j] : 0.f;
        p[u] = in ? sP[r * B + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t qa[4] = {qw[u].x, qw[u].y, qw[u].z, qw[u].w}, oa[4] = {ow[u].x, ow[u].y, ow[u].z, ow[u].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ak[2 * w] = fmaf(ds[u], __uint_as_float(qa[w] << 16), ak[2 * w]);
          ak[2 * w + 1] = fmaf(ds[u], __uint_as_float(qa[w] & 0xffff0000u), ak[2 * w + 1]);
          av[2 * w] = fmaf(p[u], __uint_as_float(oa[w] << 16), av[2 * w]);
          av[2 * w + 1] = fmaf(p[u], __uint_as_float(oa[w] & 0xffff0000u), av[2 * w + 1]);
        }
      }
    }
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      kw[w] = (uint32_t)f32_to_bf16_bits(a.sm_scale * ak[2 * w]) |
              ((uint32_t)f32_to_bf16_bits(a.sm_scale * ak[2 * w + 1]) << 16);
      vw[w] = (uint32_t)f32_to_bf16_bits(av[2 * w]) | ((uint32_t)f32_to_bf16_bits(av[2 * w + 1]) << 16);
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
  const size_t lds = (size_t)(2 * a.block * 128 + 2 * a.group * a.block * a.block) * sizeof(float);
  hipLaunchKernelGGL(own_bwd_kernel, dim3((unsigned)n_blocks, (unsigned)a.hkv), dim3(OWN_THREADS), lds, stream, a);
  return hipGetLastError();
}

}  // namespace skv
