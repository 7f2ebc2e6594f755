// Backward of Split-KV block-sparse draft attention, bf16, head_dim 128.
//
// The merged log-sum-exp of the forward is reused, so P = exp(s - LSE) is
// recomputed exactly without another softmax pass (pages: Split-KV article,
// "Split-KV's Core Mechanism": the exact aggregation is what keeps gradients
// correct).  With dS = P * (dO.v - Delta), Delta = sum_x dO * O:
//     dV_j = sum_rows P dO,   dK_j = scale * sum_rows dS q,   dQ = scale * dS K.
//
// Four launches on the caller's stream (five under the own-block mask, whose
// own keys' share runs after step 3).  No result is accumulated with atomics
// (the only atomics are the integer cursors through which workgroups claim
// work items), so the result is bitwise reproducible:
//   1. preprocess: the first partial row of every sequence (for the dQ
//      partial layout), the reset of both plans' claim cursors, and copies of
//      Q, dO, LSE (log2 units), Delta and the draft block's prefix end in
//      packed row order, so that the query tiles of both main kernels are
//      contiguous rows.
//   2. key-owner kernel (persistent workgroups of 8 waves, two per SIMD, over
//      BWD items = (sequence, KV head, key range)): 256 keys at a time, 32 per
//      wave, with the keys' K staged in LDS, their V operands and fp32 dK, dV
//      accumulators in registers, walking the 32-row query tiles that see
//      those keys (anchors are sorted, so those rows are a suffix of the draft
//      blocks); the next tile's Q, dO, LSE, Delta load while the current one
//      is computed.  S = Q K^T, dP = dO V^T (A from LDS), P and dS in
//      registers, dV += P^T dO and dK += dS^T Q (B read transposed from LDS).
//   3. query-owner kernel over the forward's items (sequence, KV head, run of
//      consecutive chunks, draft blocks), structured like the forward: 64
//      rows per wave with Q in registers and dO in LDS, K/V tiles of the run
//      through two LDS buffers; S^T = K Q^T, dP^T = V dO^T, dS^T, then
//      dQ^T += K^T dS^T, with the two 32-key halves of a tile
//      software-pipelined (one half's dS work beside the other half's MFMAs).
//      Each item writes one dQ partial for its run, in its first chunk's rows
//      (with the run length beside it), like the forward's O partial.
//   4. finalize: dQ = scale * sum of the row's run partials (and, under the
//      own-block mask, its own-block partial), bf16.
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int D = 128;
constexpr int LDS_ROW = D + 8;   // bf16 per staged row (272 bytes: conflict-free 16-byte reads)

// ---------------------------------------------------------------------------
// 1. preprocess
// ---------------------------------------------------------------------------

// First partial row of every sequence: part_base[s] = sum_{s' < s} P_s' * hq * Mq_s',
// P_s = C_s partials, plus the own-block partial under the own-block mask.
__device__ void part_base_all(const BwdArgs& a) {
  int64_t base = 0;
  for (int s = 0; s < a.n_seq; ++s) {
    a.part_base[s] = base;
    const int64_t n = a.kv_off[s + 1] - a.kv_off[s];
    base += ((n + a.chunk - 1) / a.chunk + a.own) * a.hq * (a.q_off[s + 1] - a.q_off[s]);
  }
  a.part_base[a.n_seq] = base;
}

// Packed copies for the two main kernels (16 lanes per (token, head), 8 bf16
// each): Q and dO rows, LSE in log2 units, Delta = sum_x dO * O (from the
// merged O in bf16) and the prefix end of the row's draft block, all at the
// row's packed index.
//
// The launch also resets both plans' claim cursors and, in one thread, finds
// the first partial row of every sequence (the dQ partial layout).
__global__ __launch_bounds__(256) void bwd_pack_kernel(BwdArgs a) {
  {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.kv_claim_n) a.kv_claim[t] = 0;
    if (t < a.q_claim_n) a.q_claim[t] = 0;
    if (t == 0) part_base_all(a);
  }
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int ln = threadIdx.x & 15;
  const int64_t n = a.total_q * a.hq;
  if (idx >= n) return;  // whole 16-lane groups leave together
  const int64_t t = idx / a.hq;
  const int h = (int)(idx % a.hq);
  int lo = 0, hi = a.n_seq;  // sequence of token t: q_off[lo] <= t < q_off[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.q_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int64_t q0 = a.q_off[lo], mq = a.q_off[lo + 1] - q0;
  const int64_t r = t - q0;
  const int64_t b = r / a.block, i = r % a.block;
  const int g = h / a.group, hl = h % a.group;
  const int64_t P = q0 * a.hq + (int64_t)g * a.group * mq + (b * a.group + hl) * a.block + i;

  const uint16_t* O = static_cast<const uint16_t*>(a.o) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8;
  const uint16_t* dO = static_cast<const uint16_t*>(a.dout) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8;
  const uint16_t* Qr = static_cast<const uint16_t*>(a.q) + t * a.q_st + (int64_t)h * a.q_sh + ln * 8;
  const uint4 ov = *reinterpret_cast<const uint4*>(O);
  const uint4 dv = *reinterpret_cast<const uint4*>(dO);
  const uint4 qv = *reinterpret_cast<const uint4*>(Qr);
  *reinterpret_cast<uint4*>(a.qp + P * D + ln * 8) = qv;
  *reinterpret_cast<uint4*>(a.dop + P * D + ln * 8) = dv;
  const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    sum = fmaf(__uint_as_float(ow[k] << 16), __uint_as_float(dw[k] << 16), sum);
    sum = fmaf(__uint_as_float(ow[k] & 0xffff0000u), __uint_as_float(dw[k] & 0xffff0000u), sum);
  }
  for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
  if (ln == 0) {
    const int n_ctx = (int)(a.kv_off[lo + 1] - a.kv_off[lo]);
    a.deltap[P] = sum;
    a.lsep[P] = a.lse[idx] * kLog2e;
    a.endp[P] = min(a.anchor[q0 / a.block + b] + a.end_shift, n_ctx);
  }
}

// ---------------------------------------------------------------------------
// 2. key-owner kernel: dK, dV
// ---------------------------------------------------------------------------

// Staging registers of one query tile (32 rows): each of the 512 threads moves
// 16 bytes of Q and of dO; threads 0..31 also carry their row's LSE, Delta and
// prefix end.
struct QTileRegs {
  uint4 q, o;
  float lse, delta;
  int end;
};

constexpr int KV_WAVES = 8;            // two per SIMD
constexpr int KV_THREADS = 64 * KV_WAVES;
constexpr int KV_KEYS = 32 * KV_WAVES; // keys per workgroup pass: 32 per wave
constexpr int QT = 32;                // query rows per tile

struct QTileMeta {
  float lse[QT];    // LSE of each row, log2 units (+inf for padding rows: P = 0)
  float delta[QT];
  int end[QT];      // prefix end e_b of the row (keys at or past it are masked)
};

__global__ __launch_bounds__(KV_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][QT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2][QT * LDS_ROW];
  __shared__ __attribute__((aligned(16))) QTileMeta sMeta[2];
  __shared__ __attribute__((aligned(16))) uint16_t sK[KV_KEYS * LDS_ROW];
  __shared__ int s_claim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int gi = lane >> 4, li = lane & 15;
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  uint16_t* dK = static_cast<uint16_t*>(a.dk);
  uint16_t* dV = static_cast<uint16_t*>(a.dv);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;

  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int me = plan_worker();
  int victim = me, visited = 0;
  for (;;) {
    const int64_t slot = claim_next(a.kv_worker_off, a.kv_claim, victim, visited, &s_claim, a.kv_steal);
    if (slot < 0) break;
    skv_item it = a.kv_items[slot];
    it.seq = uniform(it.seq); it.kv_head = uniform(it.kv_head); it.lo = uniform(it.lo); it.hi = uniform(it.hi);
    const int s = it.seq, g = it.kv_head;
    const int64_t q0 = uniform(a.q_off[s]);
    const int64_t mq = uniform(a.q_off[s + 1]) - q0;
    const int64_t k0 = uniform(a.kv_off[s]);
    const int n_ctx = (int)(uniform(a.kv_off[s + 1]) - k0);
    const int64_t blk0 = q0 / a.block;
    const int n_blk = (int)(mq / a.block);
    const int64_t pbase = q0 * a.hq + (int64_t)g * GB * n_blk;  // first packed row of (s, g)
    const uint16_t* Kseq = K + k0 * a.kv_st + (int64_t)g * a.kv_sh;
    const uint16_t* Vseq = V + k0 * a.kv_st + (int64_t)g * a.kv_sh;

    for (int kb = it.lo; kb < it.hi; kb += KV_KEYS) {
      const int kend = min(it.hi, kb + KV_KEYS);
      // Blocks whose prefix ends at or before kb see none of these keys.
      int b_first = 0;
      for (int b0 = 0; b0 < n_blk; b0 += 64) {
        const int b = b0 + lane;
        bool blind = false;
        if (b < n_blk) blind = min(a.anchor[blk0 + b] + a.end_shift, n_ctx) <= kb;
        b_first += __popcll(__ballot(blind));
      }
      const int nq = (n_blk - b_first) * GB;
      const int ntq = (nq + QT - 1) / QT;

      // Query tile loader: rows qt*32 + row of the visible suffix, contiguous
      // in the packed copies; padding rows read the last row and are masked.
      const int64_t vis0 = pbase + (int64_t)b_first * GB;  // packed index of the suffix's first row
      auto load_q = [&](int qt) {
        QTileRegs r;
        const int row = min(tid >> 4, nq - 1 - qt * QT);
        const int64_t off = (vis0 + qt * QT + row) * D + (tid & 15) * 8;
        r.q = *reinterpret_cast<const uint4*>(a.qp + off);
        r.o = *reinterpret_cast<const uint4*>(a.dop + off);
        r.lse = INFINITY; r.delta = 0.f; r.end = kb;
        if (tid < QT) {
          const int p = qt * QT + tid;
          const int64_t P = vis0 + min(p, nq - 1);
          const float lse = a.lsep[P];
          const float del = a.deltap[P];
          const int e = a.endp[P];
          if (p < nq) { r.lse = lse; r.delta = del; r.end = e; }
        }
        return r;
      };
      auto store_q = [&](const QTileRegs& r, int buf) {
        const int o = (tid >> 4) * LDS_ROW + (tid & 15) * 8;
        *reinterpret_cast<uint4*>(sQ[buf] + o) = r.q;
        *reinterpret_cast<uint4*>(sdO[buf] + o) = r.o;
        if (tid < QT) {
          sMeta[buf].lse[tid] = r.lse;
          sMeta[buf].delta[tid] = r.delta;
          sMeta[buf].end[tid] = r.end;
        }
      };

      // This wave's 32 keys as MFMA B operands (k = head dim); keys past the
      // context are clamped to its last key and masked.
      const int kw0 = kb + wave * 32;           // first key of this wave
      const int key_w = kw0 + l32;
      bf16x8 vreg[8];
      {
        const int kc = min(key_w, n_ctx - 1);
        const uint16_t* vp = Vseq + (int64_t)kc * a.kv_st + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) vreg[ks] = load_bf16x8(vp + ks * 16);
      }
      __syncthreads();  // every wave is done with the previous pass's K
      {
        // 256 keys x 16 chunks of 16 bytes: thread -> key tid/2 .. in 8 steps
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = tid + u * KV_THREADS;        // 0 .. 4095
          const int key = idx >> 4, ch = idx & 15;
          const int kc = min(kb + key, n_ctx - 1);
          *reinterpret_cast<uint4*>(sK + key * LDS_ROW + ch * 8) =
              *reinterpret_cast<const uint4*>(Kseq + (int64_t)kc * a.kv_st + ch * 8);
        }
      }
      f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dk_acc[i] = dv_acc[i] = f32x16{};
      const bool wave_live = kw0 < kend;        // the wave owns at least one key of the item

      if (ntq > 0) {
        QTileRegs R = load_q(0);
        __syncthreads();  // previous users of the query buffers are done
        store_q(R, 0);
        __builtin_amdgcn_s_waitcnt(0);
        if (ntq > 1) R = load_q(1);

        for (int qt = 0; qt < ntq; ++qt) {
          const int buf = qt & 1;
          if (qt > 0) {
            store_q(R, buf);                       // tile qt, loaded during tile qt-1
            if (qt + 1 < ntq) R = load_q(qt + 1);  // in flight during this tile
          }
          __syncthreads();
          if (!wave_live) continue;
          const uint16_t* bq = sQ[buf];
          const uint16_t* bo = sdO[buf];
          const QTileMeta& M = sMeta[buf];
          // 32-bit LDS addresses of this lane's transposed reads; the empty asm
          // keeps the per-read offsets as immediates.
          uint32_t qt0 = lds_addr(bq + (4 * hf + (li >> 2)) * LDS_ROW + 16 * (gi & 1) + 4 * (li & 3));
          uint32_t ot0 = lds_addr(bo + (4 * hf + (li >> 2)) * LDS_ROW + 16 * (gi & 1) + 4 * (li & 3));
          asm volatile("" : "+v"(qt0), "+v"(ot0));

          // ---- S = Q K^T and dP = dO V^T for 32 rows x this wave's 32 keys ----
          f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            if (ks & 1) asm volatile("" ::: "memory");  // bounds how far the compiler hoists the reads
            const bf16x8 qa = lds_load_bf16x8(bq + l32 * LDS_ROW + ks * 16 + hf * 8);
            const bf16x8 oa = lds_load_bf16x8(bo + l32 * LDS_ROW + ks * 16 + hf * 8);
            const bf16x8 kf = lds_load_bf16x8(sK + (wave * 32 + l32) * LDS_ROW + ks * 16 + hf * 8);
            sacc = mfma32x32x16(qa, kf, sacc);
            pacc = mfma32x32x16(oa, vreg[ks], pacc);
          }
          // ---- P = exp2(s*c - LSE2) on visible entries, dS = P (dP - Delta) ----
          // lane holds key key_w, rows 8i + 4hf + j (element 4i + j).  Rows are
          // sorted by prefix end: if the tile's first row sees all of this
          // wave's keys (and no row is padding) no entry needs masking.
          const bool full = M.end[0] >= kw0 + 32 && qt * QT + QT <= nq;
          if (!full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int4 end4 = *reinterpret_cast<const int4*>(&M.end[8 * i + 4 * hf]);
              const int ends[4] = {end4.x, end4.y, end4.z, end4.w};
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (key_w >= ends[j]) sacc[4 * i + j] = -INFINITY;
            }
          }
          // ---- dV += P^T dO, dK += dS^T Q (A from registers, B transposed from LDS) ----
#pragma unroll
          for (int kstep = 0; kstep < 2; ++kstep) {
            const int qh = kstep * 8;
            float pv[8], dv8[8];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
              const int i = (qh >> 2) + ii;
              const int r0 = 8 * i + 4 * hf;
              const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&M.lse[r0]);
              const f32x4 del4 = *reinterpret_cast<const f32x4*>(&M.delta[r0]);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float p = fast_exp2(__builtin_fmaf(sacc[4 * i + j], c, -lse4[j]));
                pv[4 * ii + j] = p;
                dv8[4 * ii + j] = p * (pacc[4 * i + j] - del4[j]);
              }
            }
            const bf16x8 pa = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
            const bf16x8 da = to_bf16x8(dv8[0], dv8[1], dv8[2], dv8[3], dv8[4], dv8[5], dv8[6], dv8[7]);
#pragma unroll
            for (int nd = 0; nd < 4; ++nd) {
              asm volatile("" ::: "memory");
              const uint32_t so = 2u * (kstep * 16 * LDS_ROW + nd * 32);
              const bf16x8 ob = lds_tr_pair(ot0 + so, ot0 + so + 2u * 8 * LDS_ROW);
              const bf16x8 qb = lds_tr_pair(qt0 + so, qt0 + so + 2u * 8 * LDS_ROW);
              dv_acc[nd] = mfma32x32x16(pa, ob, dv_acc[nd]);
              dk_acc[nd] = mfma32x32x16(da, qb, dk_acc[nd]);
            }
          }
        }
      }

      // ---- write dK (scaled) and dV for this wave's keys inside the item ----
#pragma unroll
      for (int nd = 0; nd < 4; ++nd)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kw0 + (e >> 2) * 8 + 4 * hf + (e & 3);
          if (key < kend) {
            const int64_t off = (k0 + key) * a.kv_st + (int64_t)g * a.kv_sh + nd * 32 + l32;
            dK[off] = f32_to_bf16_bits(a.sm_scale * dk_acc[nd][e]);
            dV[off] = f32_to_bf16_bits(dv_acc[nd][e]);
          }
        }
    }
  }
  record_ticks(a.kv_ticks, me, t_start);
}

// ---------------------------------------------------------------------------
// 3. query-owner kernel: per-chunk dQ partials
// ---------------------------------------------------------------------------

constexpr int KT2 = 64;                 // keys per tile of the query-owner kernel
constexpr int TILE_ELEMS = KT2 * LDS_ROW;

struct KVTileRegs {
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

__device__ __forceinline__ KVTileRegs load_kv_tile(const uint16_t* Kseq, const uint16_t* Vseq, int kb, int n_ctx,
                                                   int64_t kv_st, int tid) {
  KVTileRegs r;
  const int64_t d8 = (tid & 15) * 8;
  const int row = tid >> 4;
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

__device__ __forceinline__ void store_kv_tile(KVTileRegs r, uint16_t* sK, uint16_t* sV, int tid) {
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
void bwd_dq_kernel(BwdArgs a) {
  // Two K/V buffers: tile t+1 is stored after the barrier that ends tile t-1,
  // so one barrier per tile suffices.  dO rows of the pass live in LDS.
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2][2][TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[256 * LDS_ROW];
  __shared__ int s_claim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int gi = lane >> 4, li = lane & 15;
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;
  const uint16_t* my_dO = sdO + (wave * 64 + l32) * LDS_ROW + hf * 8;  // this lane's row, nt = 0

  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int me = plan_worker();
  int victim = me, visited = 0;
  for (;;) {
    const int64_t slot = claim_next(a.q_worker_off, a.q_claim, victim, visited, &s_claim, a.q_steal);
    if (slot < 0) break;
    skv_item it = a.q_items[slot];
    it.seq = uniform(it.seq); it.kv_head = uniform(it.kv_head); it.chunk = uniform(it.chunk);
    it.lo = uniform(it.lo); it.hi = uniform(it.hi); it.part_base = uniform(it.part_base);
    const int s = it.seq;
    const int64_t q0 = uniform(a.q_off[s]);
    const int64_t mq = uniform(a.q_off[s + 1]) - q0;
    const int64_t k0 = uniform(a.kv_off[s]);
    const int n_ctx = (int)(uniform(a.kv_off[s + 1]) - k0);
    // packed index of the item's first row: (s, kv head) block, then draft block it.lo
    const int64_t pitem = q0 * a.hq + (int64_t)it.kv_head * a.group * mq + (int64_t)it.lo * GB;
    const int nrows = (it.hi - it.lo) * GB;
    const uint16_t* Kseq = K + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
    const uint16_t* Vseq = V + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
    // keys of the item's chunks (a run of consecutive chunks: one dQ partial
    // for all of them, in the first chunk's rows, with the run length beside it)
    const int n_chunk = max(1, uniform(it.n_chunk));
    const int klo = it.chunk * a.chunk;
    const int khi = (int)min((int64_t)(it.chunk + n_chunk) * a.chunk, (int64_t)n_ctx);
    const int64_t part_base = it.part_base;
    for (int rt = 0; rt < nrows; rt += 256) {
      const int p_last = min(nrows, rt + 256) - 1;
      const int wg_hi = max(klo, min(khi, a.endp[pitem + p_last]));
      const int ntiles = (wg_hi - klo + KT2 - 1) / KT2;
      if (ntiles == 0) continue;  // no row of the pass sees the chunk: no partial to write

      __syncthreads();  // all waves are done with the previous pass's buffers (K/V and dO)
      KVTileRegs R = load_kv_tile(Kseq, Vseq, klo, n_ctx, a.kv_st, tid);
      // ---- this lane's two rows: Q as MFMA B operand, LSE, Delta; dO rows to LDS ----
      int vend[2];
      int64_t prow[2];
      bool valid[2];
      float lse2[2], del[2];
      bf16x8 qf[2][8];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int p = rt + wave * 64 + nt * 32 + l32;
        valid[nt] = p < nrows;
        const int pc = valid[nt] ? p : p_last;
        const int b = it.lo + a.fd_gb.div(pc);
        const int hl = a.fd_group.mod(a.fd_block.div(pc));
        const int64_t r = (int64_t)b * a.block + a.fd_block.mod(pc);
        const int h = it.kv_head * a.group + hl;
        const int64_t P = pitem + pc;
        const int e = a.endp[P];
        vend[nt] = valid[nt] ? max(klo, min(khi, e)) : klo;
        prow[nt] = part_base + (int64_t)h * mq + r;
        lse2[nt] = a.lsep[P];
        del[nt] = a.deltap[P];
        const uint16_t* qrow = a.qp + P * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = load_bf16x8(qrow + ks * 16);
      }
      // dO of the pass's 256 rows: thread (row tid>>4 + 16u, 16-byte column tid&15)
      uint4 dox[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int p = min(rt + (tid >> 4) + 16 * u, p_last);
        dox[u] = *reinterpret_cast<const uint4*>(a.dop + (pitem + p) * D + (tid & 15) * 8);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        *reinterpret_cast<uint4*>(sdO + ((tid >> 4) + 16 * u) * LDS_ROW + (tid & 15) * 8) = dox[u];
      store_kv_tile(R, sKV[0][0], sKV[0][1], tid);
      __builtin_amdgcn_s_waitcnt(0);  // drain before the prefetch (see the forward kernel)
      if (ntiles > 1) R = load_kv_tile(Kseq, Vseq, klo + KT2, n_ctx, a.kv_st, tid);
      const int wave_hi = wave_max_i(max(vend[0], vend[1]));
      const int wave_full = wave_min_i(min(valid[0] ? vend[0] : INT32_MAX, valid[1] ? vend[1] : INT32_MAX));

      f32x16 acc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x16{};

      for (int t = 0; t < ntiles; ++t) {
        const int kb = klo + t * KT2;
        __syncthreads();  // tile t visible; every wave is done with tile t-1's buffer
        if (t + 1 < ntiles) {
          store_kv_tile(R, sKV[(t + 1) & 1][0], sKV[(t + 1) & 1][1], tid);
          if (t + 2 < ntiles) R = load_kv_tile(Kseq, Vseq, kb + 2 * KT2, n_ctx, a.kv_st, tid);
        }
        if (kb >= wave_hi) continue;
        const uint16_t* sK = sKV[t & 1][0];
        const uint16_t* sV = sKV[t & 1][1];

        // The 64 keys are two halves of 32 (mt = 0, 1).  Within the tile the
        // halves are software-pipelined: each k step of half 1's S^T / dP^T
        // products carries part of half 0's dS work, and each step of half 0's
        // dQ products part of half 1's, so the VALU work of one half runs in
        // the shadow of the other half's MFMAs.  Every value is computed as in
        // a plain half-by-half loop; only the instruction order differs.
        auto tile = [&](auto mask_c) {
          constexpr bool MASK = decltype(mask_c)::value;  // partial tile: keys past a row's end are masked
          // dS^T = P^T (dP^T - Delta), P^T = exp2(s*c - LSE2) on visible keys,
          // for elements e0 and e0 + 1 of both row groups of half mt
          auto ds_pair = [&](int mt, int e0, f32x16 (&sacc)[2], const f32x16 (&pacc)[2]) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
              for (int e = e0; e < e0 + 2; ++e) {
                float p = fast_exp2(__builtin_fmaf(sacc[nt][e], c, -lse2[nt]));
                if (MASK) {
                  const int key = kb + mt * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
                  if (key >= vend[nt]) p = 0.f;
                }
                sacc[nt][e] = p * (pacc[nt][e] - del[nt]);
              }
          };
          // k step ks of S^T = K Q^T and dP^T = V dO^T for keys mt*32 .. +32
          auto sp_step = [&](int mt, int ks, f32x16 (&sacc)[2], f32x16 (&pacc)[2]) {
            const bf16x8 kf = lds_load_bf16x8(sK + (mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8);
            const bf16x8 vf = lds_load_bf16x8(sV + (mt * 32 + l32) * LDS_ROW + ks * 16 + hf * 8);
            sacc[0] = mfma32x32x16(kf, qf[0][ks], sacc[0]);
            sacc[1] = mfma32x32x16(kf, qf[1][ks], sacc[1]);
            pacc[0] = mfma32x32x16(vf, lds_load_bf16x8(my_dO + ks * 16), pacc[0]);
            pacc[1] = mfma32x32x16(vf, lds_load_bf16x8(my_dO + 32 * LDS_ROW + ks * 16), pacc[1]);
          };
          // dS^T of keys mt*32 + 16*half .. +16 as bf16 MFMA operands
          auto to_df = [&](const f32x16 (&sacc)[2], int half, bf16x8 (&df)[2]) {
            const int qh = half * 8;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              const f32x16& sv = sacc[nt];
              df[nt] = to_bf16x8(sv[qh + 0], sv[qh + 1], sv[qh + 2], sv[qh + 3], sv[qh + 4], sv[qh + 5],
                                 sv[qh + 6], sv[qh + 7]);
            }
          };
          // head-dim block md of dQ^T += K^T dS^T over keys mt*32 + 16*half .. +16
          // (K^T read transposed from LDS)
          auto dq_step = [&](int mt, int half, int md, const bf16x8 (&df)[2]) {
            const int key0 = (2 * mt + half) * 16 + 4 * hf + (li >> 2);
            const int col = md * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const bf16x8 kt = lds_tr_pair(sK + key0 * LDS_ROW + col, sK + (key0 + 8) * LDS_ROW + col);
            acc[md][0] = mfma32x32x16(kt, df[0], acc[md][0]);
            acc[md][1] = mfma32x32x16(kt, df[1], acc[md][1]);
          };

          f32x16 s0[2], p0[2], s1[2], p1[2];
          s0[0] = s0[1] = p0[0] = p0[1] = f32x16{};
          s1[0] = s1[1] = p1[0] = p1[1] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) sp_step(0, ks, s0, p0);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {  // half 1's scores with half 0's dS
            sp_step(1, ks, s1, p1);
            ds_pair(0, 2 * ks, s0, p0);
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {  // half 0's dQ with half 1's dS
            bf16x8 df[2];
            to_df(s0, half, df);
#pragma unroll
            for (int md = 0; md < 4; ++md) {
              dq_step(0, half, md, df);
              ds_pair(1, 2 * (half * 4 + md), s1, p1);
            }
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 df[2];
            to_df(s1, half, df);
#pragma unroll
            for (int md = 0; md < 4; ++md) dq_step(1, half, md, df);
          }
        };
        if (kb + KT2 > wave_full) tile(std::integral_constant<bool, true>{});
        else tile(std::integral_constant<bool, false>{});
      }

      // ---- the item's dQ partial (unscaled) for rows that see its keys ----
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (!valid[nt] || vend[nt] <= klo) continue;
        if (hf == 0) a.dq_run[prow[nt]] = n_chunk;
        float* op = a.dq_part + prow[nt] * D + hf * 4;
#pragma unroll
        for (int md = 0; md < 4; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 v4 = {acc[md][nt][4 * i + 0], acc[md][nt][4 * i + 1], acc[md][nt][4 * i + 2],
                        acc[md][nt][4 * i + 3]};
            *reinterpret_cast<f32x4*>(op + md * 32 + 8 * i) = v4;
          }
      }
    }
  }
  record_ticks(a.q_ticks, me, t_start);
}

// ---------------------------------------------------------------------------
// 4. finalize: dQ = scale * sum of the row's dQ partials
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdArgs a) {
  // 32 lanes per (row, head), 4 fp32 each.
  const int64_t idx = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int ln = threadIdx.x & 31;
  if (idx >= a.total_q * a.hq) return;
  const int64_t t = idx / a.hq;
  const int h = (int)(idx % a.hq);
  int lo = 0, hi = a.n_seq;  // sequence of token t: q_off[s] <= t < q_off[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.q_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int64_t q0 = a.q_off[s], mq = a.q_off[s + 1] - q0;
  const int64_t r = t - q0;
  const int n_ctx = (int)(a.kv_off[s + 1] - a.kv_off[s]);
  const int e = min(a.anchor[(q0 + r) / a.block] + a.end_shift, n_ctx);
  const int nc = (e + a.chunk - 1) / a.chunk;  // chunks the row sees
  const int64_t prow0 = a.part_base[s] + (int64_t)h * mq + r;
  const float* src = a.dq_part + prow0 * D + ln * 4;
  const int64_t cstride = (int64_t)a.hq * mq * D;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  // The chunks the row sees are covered by runs in order; each run's partial
  // sits in its first chunk's rows with the run length beside it (>= 1, so
  // the walk always ends).
  for (int cc = 0; cc < nc;) {
    sum += *reinterpret_cast<const f32x4*>(src + cc * cstride);
    cc += max(1, a.dq_run[prow0 + (int64_t)cc * a.hq * mq]);
  }
  if (a.own) {  // the own-block partial follows the sequence's chunks
    const int n_chunk = (n_ctx + a.chunk - 1) / a.chunk;
    sum += *reinterpret_cast<const f32x4*>(src + n_chunk * cstride);
  }
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16_bits(a.sm_scale * sum[0]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * sum[1]) << 16);
  pk.y = (uint32_t)f32_to_bf16_bits(a.sm_scale * sum[2]) | ((uint32_t)f32_to_bf16_bits(a.sm_scale * sum[3]) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dq) + t * a.q_st + (int64_t)h * a.q_sh + ln * 4) = pk;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int kv_workers, int q_workers, hipStream_t stream) {
  const int64_t rows = a.total_q * a.hq;
  hipError_t e;
  {
    // Packed copies, claim cursor resets and partial offsets in one launch
    // (at least one workgroup even without query rows).
    const int64_t claims = std::max(a.kv_claim_n, a.q_claim_n);
    const int64_t blocks = std::max<int64_t>(std::max<int64_t>((rows + 15) / 16, (claims + 255) / 256), 1);
    TimedLaunch t(kBwdPack, stream);
    hipLaunchKernelGGL(bwd_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    TimedLaunch t(kBwdKv, stream);
    hipLaunchKernelGGL(bwd_kv_kernel, dim3(kv_workers), dim3(KV_THREADS), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    TimedLaunch t(kBwdDq, stream);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(q_workers), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess || rows == 0) return e;
  }
  if (a.own && (e = launch_own_bwd(a, a.total_q / a.block, stream)) != hipSuccess) return e;
  TimedLaunch t(kBwdFinalize, stream);
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
