// Split-KV partial forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// One KV chunk's contribution to the attention of a range of draft blocks
// (pages: Split-KV article, "Split-KV's Core Mechanism": each KV shard stays
// local and yields a query-sized result that is later aggregated exactly).
//
// Persistent workgroups: workgroup w runs the work items the planner gave it.
// An item is (sequence, KV head g with its G query heads, chunk c, draft
// blocks [lo, hi)).  Its query rows are packed block-major as
// p = ((b - lo) * G + head) * B + token, 256 rows per pass: 4 waves x 64 rows.
// Each wave keeps its 64 Q rows in registers and the unnormalised O^T
// (128 x 64, fp32) in accumulators.  The workgroup stages 64-key K and V tiles
// through LDS; key tiles no row of the workgroup sees are never loaded.
//
// Per key tile and wave:  S^T = K Q^T (MFMA 32x32x16, K from LDS), masking of
// keys at or beyond the row's prefix end e_b, online softmax in the exp2
// domain, O^T += V^T P^T with V^T read from LDS by ds_read_b64_tr_b16 and P^T
// taken straight from the S^T accumulators (the key order inside each 16-key
// step is permuted identically on both operands).
#include "device.h"
#include "launch.h"

namespace skv {
namespace {

constexpr int D = 128;
constexpr int KT = 64;             // keys per tile
constexpr int NWAVE = 4;
constexpr int ROWS = 64 * NWAVE;   // packed query rows per pass
constexpr int LDS_ROW = D + 8;     // bf16 elements per staged key row (272 bytes)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[KT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KT * LDS_ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const int GB = a.group * a.block;

  const int64_t slot_end = a.worker_off[blockIdx.x + 1];
  for (int64_t slot = a.worker_off[blockIdx.x]; slot < slot_end; ++slot) {
    const skv_item it = a.items[slot];
    const int s = it.seq;
    const int64_t q0 = a.q_off[s];
    const int64_t mq = a.q_off[s + 1] - q0;
    const int64_t k0 = a.kv_off[s];
    const int n_ctx = (int)(a.kv_off[s + 1] - k0);
    const int64_t blk0 = q0 / a.block;
    const int klo = it.chunk * a.chunk;
    const int khi = min(klo + a.chunk, n_ctx);
    const int nrows = (it.hi - it.lo) * GB;
    const uint16_t* Kg = K + (k0 + klo) * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
    const uint16_t* Vg = V + (k0 + klo) * a.kv_st + (int64_t)it.kv_head * a.kv_sh;

    for (int rt = 0; rt < nrows; rt += ROWS) {
      // ---- this lane's two rows (S^T / O^T column l32 of each 32-row half) ----
      int vend[2];          // visible keys of the row in this chunk: [klo, vend)
      int64_t prow[2];      // partial row index
      bool valid[2];
      bf16x8 qf[2][8];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int p = rt + wave * 64 + nt * 32 + l32;
        valid[nt] = p < nrows;
        vend[nt] = klo;
        prow[nt] = 0;
        if (valid[nt]) {
          const int b = it.lo + p / GB;
          const int hl = (p / a.block) % a.group;
          const int i = p % a.block;
          const int e = min(a.anchor[blk0 + b] + a.block, n_ctx);
          vend[nt] = max(klo, min(khi, e));
          const int h = it.kv_head * a.group + hl;
          const int64_t r = (int64_t)b * a.block + i;
          prow[nt] = it.part_base + (int64_t)h * mq + r;
          const uint16_t* qp = Q + (q0 + r) * a.q_st + (int64_t)h * a.q_sh + hf * 8;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = load_bf16x8(qp + ks * 16);
        } else {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = bf16x8{};
        }
      }
      const int wave_hi = wave_max_i(max(vend[0], vend[1]));
      const int wave_full = wave_min_i(min(valid[0] ? vend[0] : INT32_MAX, valid[1] ? vend[1] : INT32_MAX));
      // Anchors are sorted, so the last row of the pass has the largest prefix end.
      const int p_last = min(nrows, rt + ROWS) - 1;
      const int b_last = it.lo + p_last / GB;
      const int wg_hi = max(klo, min(khi, min(a.anchor[blk0 + b_last] + a.block, n_ctx)));

      float m[2] = {-INFINITY, -INFINITY};  // running row max (log2 units)
      float l[2] = {0.f, 0.f};              // this lane-half's running row sum
      f32x16 acc_o[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i][0] = acc_o[i][1] = f32x16{};

      for (int kb = klo; kb < wg_hi; kb += KT) {
        __syncthreads();  // previous tile fully consumed
        // ---- stage K and V tile [kb, kb+64) through LDS (zeros past the context) ----
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ci = tid + 256 * u;
          const int key = ci >> 4, dc = ci & 15;
          uint4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
          if (kb + key < n_ctx) {
            kx = *reinterpret_cast<const uint4*>(Kg + (int64_t)(kb - klo + key) * a.kv_st + dc * 8);
            vx = *reinterpret_cast<const uint4*>(Vg + (int64_t)(kb - klo + key) * a.kv_st + dc * 8);
          }
          *reinterpret_cast<uint4*>(&sK[key * LDS_ROW + dc * 8]) = kx;
          *reinterpret_cast<uint4*>(&sV[key * LDS_ROW + dc * 8]) = vx;
        }
        __syncthreads();
        if (kb >= wave_hi) continue;  // no row of this wave sees the tile

        // ---- S^T = K Q^T ----
        f32x16 sacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sacc[i][0] = sacc[i][1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 kf = lds_load_bf16x8(&sK[(mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8]);
            sacc[mt][0] = mfma32x32x16(kf, qf[0][ks], sacc[mt][0]);
            sacc[mt][1] = mfma32x32x16(kf, qf[1][ks], sacc[mt][1]);
          }
        }
        // ---- mask, online softmax ----
        const bool need_mask = kb + KT > wave_full;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float rmax = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float x = sacc[mt][nt][e] * a.scale_log2;
              if (need_mask) {
                const int key = kb + mt * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
                if (key >= vend[nt]) x = -INFINITY;
              }
              sacc[mt][nt][e] = x;
              rmax = fmaxf(rmax, x);
            }
          }
          rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
          const float m_new = fmaxf(m[nt], rmax);
          const float msafe = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = fast_exp2(m[nt] - msafe);
          m[nt] = m_new;
          float psum = 0.f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float pe = fast_exp2(sacc[mt][nt][e] - msafe);
              sacc[mt][nt][e] = pe;
              psum += pe;
            }
          }
          l[nt] = l[nt] * alpha + psum;
#pragma unroll
          for (int md = 0; md < 4; ++md) acc_o[md][nt] *= alpha;
        }
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          const int mt = kstep >> 1, qh = (kstep & 1) * 8;
          bf16x8 pf[2];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const f32x16& sv = sacc[mt][nt];
            pf[nt] = to_bf16x8(sv[qh + 0], sv[qh + 1], sv[qh + 2], sv[qh + 3], sv[qh + 4], sv[qh + 5], sv[qh + 6],
                               sv[qh + 7]);
          }
          const int gi = lane >> 4, li = lane & 15;
          const int key0 = kstep * 16 + 4 * hf + (li >> 2);
#pragma unroll
          for (int md = 0; md < 4; ++md) {
            const int col = md * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const bf16x8 vf = lds_tr_pair(&sV[key0 * LDS_ROW + col], &sV[(key0 + 8) * LDS_ROW + col]);
            acc_o[md][0] = mfma32x32x16(vf, pf[0], acc_o[md][0]);
            acc_o[md][1] = mfma32x32x16(vf, pf[1], acc_o[md][1]);
          }
        }
      }

      // ---- epilogue: unnormalised O_c, row max and log-sum-exp (natural log) ----
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float lt = l[nt] + __shfl_xor(l[nt], 32);
        if (!valid[nt]) continue;
        const bool seen = lt > 0.f;
        if (hf == 0) {
          a.m_part[prow[nt]] = seen ? m[nt] * kLn2 : -INFINITY;
          a.lse_part[prow[nt]] = seen ? (m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
        }
        if (seen) {
          float* op = a.o_part + prow[nt] * D + hf * 4;
#pragma unroll
          for (int md = 0; md < 4; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              f32x4 v4 = {acc_o[md][nt][4 * i + 0], acc_o[md][nt][4 * i + 1], acc_o[md][nt][4 * i + 2],
                          acc_o[md][nt][4 * i + 3]};
              *reinterpret_cast<f32x4*>(op + md * 32 + 8 * i) = v4;
            }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int n_workers, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(n_workers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
