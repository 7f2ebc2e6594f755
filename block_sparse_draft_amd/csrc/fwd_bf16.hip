// Split-KV partial forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// One KV chunk's contribution to the attention of a range of draft blocks
// (pages: Split-KV article, "Split-KV's Core Mechanism": each KV shard stays
// local and yields a query-sized result that is later aggregated exactly).
//
// Persistent workgroups: each runs the work items the planner gave its worker,
// then claims whatever is left on other workers' lists.
// An item is (sequence, KV head g with its G query heads, chunk c, draft
// blocks [lo, hi)).  Its query rows are packed block-major as
// p = ((b - lo) * G + head) * B + token, 256 rows per pass: 4 waves x 64 rows.
// Each wave keeps its 64 Q rows in registers and the unnormalised O^T
// (128 x 64, fp32) in accumulators.  Only the 64-key tiles that some row of
// the pass sees are visited; the rest of the chunk is never read.
//
// Pipeline: K/V tiles rotate through three LDS buffers.  While tile t is
// computed, tile t+1 sits in LDS and tile t+2 is in flight from memory into
// registers, so a single barrier per tile suffices and load latency hides
// behind a tile of MFMA work.
//
// Per key tile and wave:  S^T = K Q^T (MFMA 32x32x16, K from LDS), masking of
// keys at or beyond the row's prefix end e_b (partial tiles only), online
// softmax in the exp2 domain with lazy rescaling (the reference maximum only
// moves when the true maximum exceeds it by 2^8; the output is corrected to
// the true maximum once per item), O^T += V^T P^T with V^T read from LDS by
// ds_read_b64_tr_b16 and P^T taken straight from the S^T accumulators (the key
// order inside each 16-key step is permuted identically on both operands).
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int D = 128;
constexpr int KT = 64;             // keys per tile
constexpr int NWAVE = 4;
constexpr int ROWS = 64 * NWAVE;   // packed query rows per pass
constexpr int LDS_ROW = D + 8;     // bf16 per staged key row (272 bytes: conflict-free 16-byte reads)
constexpr int TILE_ELEMS = KT * LDS_ROW;
constexpr int NBUF = 3;
constexpr float LAZY_LOG2 = 8.f;   // rescale only when the max grows by more than 2^8

// Staging registers of one K/V tile: each thread moves 4 x 16 bytes of K and of V.
struct TileRegs {
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

// Issue the loads of key tile [kb, kb+64) (sequence-relative).  Keys past the
// context are clamped to its last key: they are masked for every row.
__device__ __forceinline__ TileRegs load_tile(const uint16_t* Kseq, const uint16_t* Vseq, int kb, int n_ctx,
                                              int64_t kv_st, int tid) {
  TileRegs r;
  const int64_t d8 = (tid & 15) * 8;
  const int row = tid >> 4;  // 16 rows per 256 threads; rows row, row+16, row+32, row+48
  const int64_t o0 = (int64_t)min(kb + row, n_ctx - 1) * kv_st + d8;
  const int64_t o1 = (int64_t)min(kb + row + 16, n_ctx - 1) * kv_st + d8;
  const int64_t o2 = (int64_t)min(kb + row + 32, n_ctx - 1) * kv_st + d8;
  const int64_t o3 = (int64_t)min(kb + row + 48, n_ctx - 1) * kv_st + d8;
  r.k0 = *reinterpret_cast<const uint4*>(Kseq + o0);
  r.k1 = *reinterpret_cast<const uint4*>(Kseq + o1);
  r.k2 = *reinterpret_cast<const uint4*>(Kseq + o2);
  r.k3 = *reinterpret_cast<const uint4*>(Kseq + o3);
  r.v0 = *reinterpret_cast<const uint4*>(Vseq + o0);
  r.v1 = *reinterpret_cast<const uint4*>(Vseq + o1);
  r.v2 = *reinterpret_cast<const uint4*>(Vseq + o2);
  r.v3 = *reinterpret_cast<const uint4*>(Vseq + o3);
  return r;
}

__device__ __forceinline__ void store_tile(TileRegs r, uint16_t* sK, uint16_t* sV, int tid) {
  const int o = (tid >> 4) * LDS_ROW + (tid & 15) * 8;
  constexpr int R16 = 16 * LDS_ROW;
  *reinterpret_cast<uint4*>(sK + o) = r.k0;
  *reinterpret_cast<uint4*>(sK + o + R16) = r.k1;
  *reinterpret_cast<uint4*>(sK + o + 2 * R16) = r.k2;
  *reinterpret_cast<uint4*>(sK + o + 3 * R16) = r.k3;
  *reinterpret_cast<uint4*>(sV + o) = r.v0;
  *reinterpret_cast<uint4*>(sV + o + R16) = r.v1;
  *reinterpret_cast<uint4*>(sV + o + 2 * R16) = r.v2;
  *reinterpret_cast<uint4*>(sV + o + 3 * R16) = r.v3;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sKV[NBUF][2][TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int gi = lane >> 4, li = lane & 15;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;

  __shared__ int s_claim;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int me = plan_worker();
  int victim = me, visited = 0;
  for (;;) {
    const int64_t slot = claim_next(a.worker_off, a.claim, victim, visited, &s_claim, a.steal);
    if (slot < 0) break;
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
    const uint16_t* Kseq = K + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
    const uint16_t* Vseq = V + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;

    for (int rt = 0; rt < nrows; rt += ROWS) {
      // Anchors are sorted, so the last row of the pass has the largest prefix end.
      const int p_last = min(nrows, rt + ROWS) - 1;
      const int wg_hi = max(klo, min(khi, min(a.anchor[blk0 + it.lo + a.fd_gb.div(p_last)] + a.block, n_ctx)));
      const int ntiles = (wg_hi - klo + KT - 1) / KT;

      // ---- start the K/V pipeline around the loads of this lane's two Q rows ----
      TileRegs R;
      if (ntiles > 0) {
        __syncthreads();  // all waves are done with the previous pass's buffers
        R = load_tile(Kseq, Vseq, klo, n_ctx, a.kv_st, tid);
      }
      int vend[2];          // visible keys of the row in this chunk: [klo, vend)
      int64_t prow[2];      // partial row index
      bool valid[2];
      bf16x8 qf[2][8];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int p = rt + wave * 64 + nt * 32 + l32;
        valid[nt] = p < nrows;
        const int pc = valid[nt] ? p : p_last;  // clamp: loads stay in bounds, results unused
        const int b = it.lo + a.fd_gb.div(pc);
        const int hl = a.fd_group.mod(a.fd_block.div(pc));
        const int64_t r = (int64_t)b * a.block + a.fd_block.mod(pc);
        const int h = it.kv_head * a.group + hl;
        const int e = min(a.anchor[blk0 + b] + a.block, n_ctx);
        vend[nt] = valid[nt] ? max(klo, min(khi, e)) : klo;
        prow[nt] = it.part_base + (int64_t)h * mq + r;
        const uint16_t* qp = Q + (q0 + r) * a.q_st + (int64_t)h * a.q_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = load_bf16x8(qp + ks * 16);
      }
      if (ntiles > 0) store_tile(R, sKV[0][0], sKV[0][1], tid);
      // Drain every outstanding load (Q included) before the prefetch starts, so
      // that inside the tile loop only the prefetch itself is in flight and no
      // wait for it is needed before the S = K Q^T products.
      __builtin_amdgcn_s_waitcnt(0);
      if (ntiles > 1) R = load_tile(Kseq, Vseq, klo + KT, n_ctx, a.kv_st, tid);
      const int wave_hi = wave_max_i(max(vend[0], vend[1]));
      const int wave_full = wave_min_i(min(valid[0] ? vend[0] : INT32_MAX, valid[1] ? vend[1] : INT32_MAX));

      float m_true[2] = {-INFINITY, -INFINITY};  // running row max of raw scores
      float m_ref[2] = {-INFINITY, -INFINITY};   // max the exponentials are taken against
      float l[2] = {0.f, 0.f};                   // this lane-half's running row sum
      f32x16 acc_o[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i][0] = acc_o[i][1] = f32x16{};

      for (int t = 0; t < ntiles; ++t) {
        const int kb = klo + t * KT;
        if (t + 1 < ntiles) {
          store_tile(R, sKV[(t + 1) % NBUF][0], sKV[(t + 1) % NBUF][1], tid);
          if (t + 2 < ntiles) R = load_tile(Kseq, Vseq, kb + 2 * KT, n_ctx, a.kv_st, tid);
        }
        __syncthreads();
        if (kb >= wave_hi) continue;  // no row of this wave sees the tile
        const uint16_t* sK = sKV[t % NBUF][0];
        const uint16_t* sV = sKV[t % NBUF][1];

        // ---- S^T = K Q^T (raw scores) ----
        f32x16 sacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sacc[i][0] = sacc[i][1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 kf = lds_load_bf16x8(sK + (mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8);
            sacc[mt][0] = mfma32x32x16(kf, qf[0][ks], sacc[mt][0]);
            sacc[mt][1] = mfma32x32x16(kf, qf[1][ks], sacc[mt][1]);
          }
        }
        // ---- mask keys at or past the row's prefix end (partial tiles only) ----
        if (kb + KT > wave_full) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int key = kb + mt * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
                if (key >= vend[nt]) sacc[mt][nt][e] = -INFINITY;
              }
        }
        // ---- row max; lazy rescale when some row's max grew past 2^8 ----
        bool grow = false;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float r0 = fmaxf(sacc[0][nt][0], sacc[1][nt][0]);
#pragma unroll
          for (int e = 1; e < 16; ++e) r0 = fmaxf(r0, fmaxf(sacc[0][nt][e], sacc[1][nt][e]));
          r0 = fmaxf(r0, __shfl_xor(r0, 32));
          m_true[nt] = fmaxf(m_true[nt], r0);
          grow |= (m_true[nt] - m_ref[nt]) * c > LAZY_LOG2;  // false while both are -inf
        }
        if (__any(grow)) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float alpha = fast_exp2((m_ref[nt] - m_true[nt]) * c);  // 0 from -inf, 1 if unchanged
            const bool keep = m_true[nt] == -INFINITY;
            m_ref[nt] = m_true[nt];
            if (!keep) {
              l[nt] *= alpha;
#pragma unroll
              for (int md = 0; md < 4; ++md) acc_o[md][nt] *= alpha;
            }
          }
        }
        // ---- P = exp2(s*c - m_ref*c) ----
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float mc = m_ref[nt] == -INFINITY ? 0.f : m_ref[nt] * c;
          float psum = 0.f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float pe = fast_exp2(__builtin_fmaf(sacc[mt][nt][e], c, -mc));
              sacc[mt][nt][e] = pe;
              psum += pe;
            }
          l[nt] += psum;
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
          const int key0 = kstep * 16 + 4 * hf + (li >> 2);
#pragma unroll
          for (int md = 0; md < 4; ++md) {
            const int col = md * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const bf16x8 vf = lds_tr_pair(sV + key0 * LDS_ROW + col, sV + (key0 + 8) * LDS_ROW + col);
            acc_o[md][0] = mfma32x32x16(vf, pf[0], acc_o[md][0]);
            acc_o[md][1] = mfma32x32x16(vf, pf[1], acc_o[md][1]);
          }
        }
      }

      // ---- epilogue: unnormalised O_c against the true row max, max and log-sum-exp ----
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float lt = l[nt] + __shfl_xor(l[nt], 32);
        if (!valid[nt]) continue;
        const bool seen = lt > 0.f;
        const float fix = seen ? fast_exp2((m_ref[nt] - m_true[nt]) * c) : 1.f;
        lt *= fix;
        if (hf == 0) {
          a.m_part[prow[nt]] = seen ? m_true[nt] * a.sm_scale : -INFINITY;
          a.lse_part[prow[nt]] = seen ? (m_true[nt] * c + __log2f(lt)) * kLn2 : -INFINITY;
        }
        if (seen) {
          float* op = a.o_part + prow[nt] * D + hf * 4;
#pragma unroll
          for (int md = 0; md < 4; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              f32x4 v4 = {acc_o[md][nt][4 * i + 0] * fix, acc_o[md][nt][4 * i + 1] * fix,
                          acc_o[md][nt][4 * i + 2] * fix, acc_o[md][nt][4 * i + 3] * fix};
              *reinterpret_cast<f32x4*>(op + md * 32 + 8 * i) = v4;
            }
        }
      }
    }
  }
  record_ticks(a.ticks, me, t_start);
}

// Resets the per-worker claim cursors of a plan before a launch.
__global__ void claim_reset_kernel(int32_t* claim, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) claim[i] = 0;
}

}  // namespace

hipError_t launch_claim_reset(int32_t* claim, int n_workers, hipStream_t stream) {
  TimedLaunch t(kClaimReset, stream);
  hipLaunchKernelGGL(claim_reset_kernel, dim3((n_workers + 255) / 256), dim3(256), 0, stream, claim, n_workers);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int n_workers, hipStream_t stream) {
  TimedLaunch t(kFwdBf16, stream);
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(n_workers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
