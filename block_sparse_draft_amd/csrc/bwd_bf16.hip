// Backward of Split-KV block-sparse draft attention, bf16, head_dim 128.
//
// The merged log-sum-exp of the forward is reused, so P = exp(s - LSE) is
// recomputed exactly without another softmax pass (pages: Split-KV article,
// "Split-KV's Core Mechanism": the exact aggregation is what keeps gradients
// correct).  Three launches on the caller's stream:
//   1. preprocess: Delta = sum_x dO*O per (query row, head); zero the fp32 dQ
//      accumulator.
//   2. main (persistent workgroups over BWD items = (sequence, KV head, key
//      range)): each workgroup owns 128 keys at a time (32 per wave), keeps
//      their K, V operands and the dK, dV accumulators in registers, and
//      walks the 64-row query tiles that see those keys.  Anchors are sorted,
//      so the rows that see keys >= kb are the blocks with e_b > kb: a suffix.
//      Per query tile:  S = Q K^T and dP = dO V^T (A from LDS), P and dS in
//      registers, dV += P^T dO and dK += dS^T Q (B read transposed from LDS),
//      dS^T staged in LDS, dQ += dS K split over the 4 waves and added to the
//      fp32 accumulator with hardware float atomics.
//   3. finalize: dQ = sm_scale * accumulator, rounded to bf16.
#include "device.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int D = 128;
constexpr int KT = 128;          // keys per workgroup tile (32 per wave)
constexpr int QT = 64;           // query rows per tile
constexpr int LDS_ROW = D + 8;   // bf16 per staged row of Q, dO, K (272 bytes)
constexpr int DS_ROW = QT + 8;   // bf16 per staged key row of dS^T (144 bytes)

__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  // 16 lanes per (row, head), 8 bf16 each.
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int ln = threadIdx.x & 15;
  const int64_t n = a.total_q * a.hq;
  if (idx >= n) return;  // whole 16-lane groups leave together
  const int64_t t = idx / a.hq;
  const int h = (int)(idx % a.hq);
  const uint16_t* O = static_cast<const uint16_t*>(a.o) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8;
  const uint16_t* dO = static_cast<const uint16_t*>(a.dout) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8;
  const uint4 ov = *reinterpret_cast<const uint4*>(O);
  const uint4 dv = *reinterpret_cast<const uint4*>(dO);
  const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sum = fmaf(__uint_as_float(ow[i] << 16), __uint_as_float(dw[i] << 16), sum);
    sum = fmaf(__uint_as_float(ow[i] & 0xffff0000u), __uint_as_float(dw[i] & 0xffff0000u), sum);
  }
  for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
  if (ln == 0) a.delta[idx] = sum;
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float* acc = a.dq_acc + idx * D + ln * 8;
  *reinterpret_cast<f32x4*>(acc) = z;
  *reinterpret_cast<f32x4*>(acc + 4) = z;
}

__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int ln = threadIdx.x & 15;
  if (idx >= a.total_q * a.hq) return;
  const int64_t t = idx / a.hq;
  const int h = (int)(idx % a.hq);
  const float* acc = a.dq_acc + idx * D + ln * 8;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(acc);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(acc + 4);
  uint4 pk;
  pk.x = (uint32_t)f32_to_bf16_bits(a.sm_scale * x0[0]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * x0[1]) << 16);
  pk.y = (uint32_t)f32_to_bf16_bits(a.sm_scale * x0[2]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * x0[3]) << 16);
  pk.z = (uint32_t)f32_to_bf16_bits(a.sm_scale * x1[0]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * x1[1]) << 16);
  pk.w = (uint32_t)f32_to_bf16_bits(a.sm_scale * x1[2]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * x1[3]) << 16);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.dq) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8) = pk;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[KT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[QT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[QT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[KT * DS_ROW];
  __shared__ __attribute__((aligned(16))) float sLse[QT];
  __shared__ __attribute__((aligned(16))) float sDelta[QT];
  __shared__ __attribute__((aligned(16))) int sEnd[QT];
  __shared__ int64_t sAcc[QT];  // dq_acc row of each query row, -1 if none

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int gi = lane >> 4, li = lane & 15;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const uint16_t* dO = static_cast<const uint16_t*>(a.dout);
  uint16_t* dK = static_cast<uint16_t*>(a.dk);
  uint16_t* dV = static_cast<uint16_t*>(a.dv);
  const int GB = a.group * a.block;

  const int64_t slot_end = a.worker_off[blockIdx.x + 1];
  for (int64_t slot = a.worker_off[blockIdx.x]; slot < slot_end; ++slot) {
    const skv_item it = a.items[slot];
    const int s = it.seq, g = it.kv_head;
    const int64_t q0 = a.q_off[s];
    const int64_t k0 = a.kv_off[s];
    const int n_ctx = (int)(a.kv_off[s + 1] - k0);
    const int64_t blk0 = q0 / a.block;
    const int n_blk = (int)((a.q_off[s + 1] - q0) / a.block);

    for (int kb = it.lo; kb < it.hi; kb += KT) {
      const int kend = min(it.hi, kb + KT);
      // Blocks whose prefix ends at or before kb see none of these keys.
      int b_first = 0;
      for (int b0 = 0; b0 < n_blk; b0 += 64) {
        const int b = b0 + lane;
        const bool blind = b < n_blk && min(a.anchor[blk0 + b] + a.block, n_ctx) <= kb;
        b_first += __popcll(__ballot(blind));
      }
      const int nq = (n_blk - b_first) * GB;

      // This wave's 32 keys: K and V rows as MFMA B operands (k = head dim).
      const int key_w = kb + wave * 32 + l32;
      bf16x8 kreg[8], vreg[8];
      {
        const bool in = key_w < n_ctx;
        const uint16_t* kp = K + (k0 + key_w) * a.kv_st + (int64_t)g * a.kv_sh + hf * 8;
        const uint16_t* vp = V + (k0 + key_w) * a.kv_st + (int64_t)g * a.kv_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          kreg[ks] = in ? load_bf16x8(kp + ks * 16) : bf16x8{};
          vreg[ks] = in ? load_bf16x8(vp + ks * 16) : bf16x8{};
        }
      }
      f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dk_acc[i] = dv_acc[i] = f32x16{};

      if (nq > 0) {
        __syncthreads();  // previous users of sK are done
        // K tile [kb, kb + 128) for the dQ product
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int ci = tid + 256 * u;
          const int key = ci >> 4, dc = ci & 15;
          uint4 kx = {0, 0, 0, 0};
          if (kb + key < n_ctx)
            kx = *reinterpret_cast<const uint4*>(K + (k0 + kb + key) * a.kv_st + (int64_t)g * a.kv_sh + dc * 8);
          *reinterpret_cast<uint4*>(&sK[key * LDS_ROW + dc * 8]) = kx;
        }
      }

      for (int qt = 0; qt < nq; qt += QT) {
        __syncthreads();  // sQ, sdO, sdS of the previous tile consumed
        // ---- stage the query tile: Q, dO rows, LSE (log2 units), Delta, prefix end ----
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = tid + 256 * u;
          const int row = ci >> 4, dc = ci & 15;
          const int p = qt + row;
          uint4 qx = {0, 0, 0, 0}, ox = {0, 0, 0, 0};
          if (p < nq) {
            const int b = b_first + p / GB;
            const int h = g * a.group + (p / a.block) % a.group;
            const int64_t t = q0 + (int64_t)b * a.block + p % a.block;
            qx = *reinterpret_cast<const uint4*>(Q + t * a.q_st + (int64_t)h * a.q_sh + dc * 8);
            ox = *reinterpret_cast<const uint4*>(dO + t * a.q_st + (int64_t)h * a.q_sh + dc * 8);
          }
          *reinterpret_cast<uint4*>(&sQ[row * LDS_ROW + dc * 8]) = qx;
          *reinterpret_cast<uint4*>(&sdO[row * LDS_ROW + dc * 8]) = ox;
        }
        if (tid < QT) {
          const int p = qt + tid;
          if (p < nq) {
            const int b = b_first + p / GB;
            const int h = g * a.group + (p / a.block) % a.group;
            const int64_t t = q0 + (int64_t)b * a.block + p % a.block;
            const int64_t r = t * a.hq + h;
            sLse[tid] = a.lse[r] * kLog2e;
            sDelta[tid] = a.delta[r];
            sEnd[tid] = min(min(a.anchor[blk0 + b] + a.block, n_ctx), kend);
            sAcc[tid] = r;
          } else {
            sLse[tid] = INFINITY;  // P = 0
            sDelta[tid] = 0.f;
            sEnd[tid] = 0;
            sAcc[tid] = -1;
          }
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T for 64 rows x this wave's 32 keys ----
        f32x16 sacc[2], pacc[2];
        sacc[0] = sacc[1] = pacc[0] = pacc[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 qa = lds_load_bf16x8(&sQ[(mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8]);
            const bf16x8 oa = lds_load_bf16x8(&sdO[(mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8]);
            sacc[mt] = mfma32x32x16(qa, kreg[ks], sacc[mt]);
            pacc[mt] = mfma32x32x16(oa, vreg[ks], pacc[mt]);
          }
        }
        // ---- P = exp2(s*log2e*scale - LSE2) on visible entries, dS = P (dP - Delta) ----
        // lane holds key key_w, rows mt*32 + 8i + 4hf + j (element 4i + j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r0 = mt * 32 + 8 * i + 4 * hf;
            const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&sLse[r0]);
            const f32x4 del4 = *reinterpret_cast<const f32x4*>(&sDelta[r0]);
            const int4 end4 = *reinterpret_cast<const int4*>(&sEnd[r0]);
            const int ends[4] = {end4.x, end4.y, end4.z, end4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int e = 4 * i + j;
              float p = fast_exp2(sacc[mt][e] * a.scale_log2 - lse4[j]);
              if (key_w >= ends[j]) p = 0.f;
              sacc[mt][e] = p;
              pacc[mt][e] = p * (pacc[mt][e] - del4[j]);
            }
          }
        }
        // ---- dV += P^T dO, dK += dS^T Q (A from registers, B transposed from LDS) ----
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          const int mt = kstep >> 1, qh = (kstep & 1) * 8;
          const f32x16& ps = sacc[mt];
          const f32x16& ds = pacc[mt];
          const bf16x8 pa = to_bf16x8(ps[qh], ps[qh + 1], ps[qh + 2], ps[qh + 3], ps[qh + 4], ps[qh + 5], ps[qh + 6],
                                      ps[qh + 7]);
          const bf16x8 da = to_bf16x8(ds[qh], ds[qh + 1], ds[qh + 2], ds[qh + 3], ds[qh + 4], ds[qh + 5], ds[qh + 6],
                                      ds[qh + 7]);
          const int row0 = kstep * 16 + 4 * hf + (li >> 2);
#pragma unroll
          for (int nd = 0; nd < 4; ++nd) {
            const int col = nd * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const bf16x8 ob = lds_tr_pair(&sdO[row0 * LDS_ROW + col], &sdO[(row0 + 8) * LDS_ROW + col]);
            const bf16x8 qb = lds_tr_pair(&sQ[row0 * LDS_ROW + col], &sQ[(row0 + 8) * LDS_ROW + col]);
            dv_acc[nd] = mfma32x32x16(pa, ob, dv_acc[nd]);
            dk_acc[nd] = mfma32x32x16(da, qb, dk_acc[nd]);
          }
        }
        // ---- stage dS^T (bf16) in LDS: row key, columns = query rows ----
        {
          const int krow = wave * 32 + l32;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& ds = pacc[mt];
              uint2 pk;
              pk.x = (uint32_t)f32_to_bf16_bits(ds[4 * i]) | ((uint32_t)f32_to_bf16_bits(ds[4 * i + 1]) << 16);
              pk.y = (uint32_t)f32_to_bf16_bits(ds[4 * i + 2]) | ((uint32_t)f32_to_bf16_bits(ds[4 * i + 3]) << 16);
              *reinterpret_cast<uint2*>(&sdS[krow * DS_ROW + mt * 32 + 8 * i + 4 * hf]) = pk;
            }
        }
        __syncthreads();
        // ---- dQ (64 rows x 32 head dims of this wave) += dS K over the 128 keys ----
        f32x16 qacc[2];
        qacc[0] = qacc[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int key0 = ks * 16 + 4 * hf + (li >> 2);
          const int kcol = wave * 32 + 16 * (gi & 1) + 4 * (li & 3);
          const bf16x8 kb8 = lds_tr_pair(&sK[key0 * LDS_ROW + kcol], &sK[(key0 + 8) * LDS_ROW + kcol]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const int rcol = mt * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const bf16x8 da = lds_tr_pair(&sdS[key0 * DS_ROW + rcol], &sdS[(key0 + 8) * DS_ROW + rcol]);
            qacc[mt] = mfma32x32x16(da, kb8, qacc[mt]);
          }
        }
        // lane holds head dim wave*32 + l32 of rows mt*32 + 8i + 4hf + j
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = mt * 32 + (e >> 2) * 8 + 4 * hf + (e & 3);
            const int64_t r = sAcc[row];
            if (r >= 0) unsafeAtomicAdd(a.dq_acc + r * D + wave * 32 + l32, qacc[mt][e]);
          }
      }

      // ---- write dK (scaled) and dV for the keys of this tile inside the item ----
#pragma unroll
      for (int nd = 0; nd < 4; ++nd)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + wave * 32 + (e >> 2) * 8 + 4 * hf + (e & 3);
          if (key < kend) {
            const int64_t off = (k0 + key) * a.kv_st + (int64_t)g * a.kv_sh + nd * 32 + l32;
            dK[off] = f32_to_bf16_bits(a.sm_scale * dk_acc[nd][e]);
            dV[off] = f32_to_bf16_bits(dv_acc[nd][e]);
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int n_workers, hipStream_t stream) {
  const int64_t rows = a.total_q * a.hq;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_main_kernel, dim3(n_workers), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) return e;
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
