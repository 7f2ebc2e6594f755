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
//      registers, dV^T += dO^T P and dK^T += Q^T dS (A read transposed from
//      LDS), so each lane ends with runs of consecutive head-dim values of one
//      key and dK, dV leave as 16-byte stores.  The exponentials of P are
//      taken between the dP products and half of dS between the dV/dK
//      products, so that this VALU work issues while the matrix core runs.
//   3. query-owner kernel over the forward's items (sequence, KV head, run of
//      consecutive chunks, draft blocks), structured like the forward: 8
//      waves (two per SIMD, so one wave's LDS waits and dS arithmetic overlap
//      the other's MFMA work), 32 rows per wave with Q and dO in registers,
//      K/V tiles of the run through three LDS buffers; per 32-key half
//      S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T.  Each item
//      writes one dQ partial for its run, in its first chunk's rows (with the
//      run length beside it), like the forward's O partial.
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
// Tiles read both row-major (16-byte operand reads of 16 consecutive rows) and
// transposed (ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes per 32 lanes)
// are staged in 320-byte rows whose 16-byte chunks are XOR-swizzled by bits
// 2..3 of the row (chunk c of row r sits at c ^ ((r >> 2) & 3)): measured with
// the LDS bank-conflict counter, both kinds of read are then conflict-free (at
// 272 bytes the transposed reads collide, at 320 unswizzled the row reads).
constexpr int LDS_ROW_SW = D + 32;

// Swizzled element offsets of one lane's reads in such a tile.  Row-major
// operand (row l32 of a 32-row block, chunk 2 ks + hf, swizzle f = (l32/4)%4):
// chunk 2 (ks ^ (f / 2)) + (hf ^ f % 2), so row_off[ks % 2] + 16 (ks & ~1).
// Transposed operand (rows 16 j + 4 hf + li / 4 and 8 rows further, columns
// 32 md + 16 (gi % 2) + 4 (li % 4)): swizzles hf and hf + 2, so
// tr_off[0|1] + 16 j * LDS_ROW_SW + 32 md.
struct SwizzledOffsets {
  int row_off[2], tr_off[2];
};
__device__ __forceinline__ SwizzledOffsets swizzled_offsets(int lane) {
  const int l32 = lane & 31, hf = lane >> 5, gi = lane >> 4, li = lane & 15;
  SwizzledOffsets o;
  const int f = (l32 >> 2) & 3;
#pragma unroll
  for (int k = 0; k < 2; ++k) o.row_off[k] = l32 * LDS_ROW_SW + 16 * (k ^ (f >> 1)) + 8 * (hf ^ (f & 1));
  const int c1 = (2 * (gi & 1) + ((li & 3) >> 1)) ^ hf;
  o.tr_off[0] = (4 * hf + (li >> 2)) * LDS_ROW_SW + 8 * c1 + 4 * (li & 1);
  o.tr_off[1] = (4 * hf + (li >> 2) + 8) * LDS_ROW_SW + 8 * (c1 ^ 2) + 4 * (li & 1);
  return o;
}
// Element offset of thread tid's 16-byte store into such a tile: row
// tid / 16 (+ 16 u, 32 u: same swizzle), chunk tid % 16.
__device__ __forceinline__ int swizzled_store_off(int tid) {
  return (tid >> 4) * LDS_ROW_SW + ((tid & 15) ^ ((tid >> 6) & 3)) * 8;
}

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

// The lane's index, recomputed where it is called (v_mbcnt): values derived
// from it are then formed in place rather than hoisted and kept in scratch.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
constexpr int KV_WAVES = 8;            // two per SIMD
constexpr int KV_THREADS = 64 * KV_WAVES;
constexpr int KV_KEYS = 32 * KV_WAVES; // keys per workgroup pass: 32 per wave
constexpr int QT = 32;                // query rows per tile

struct QTileMeta {
  float lse[QT];    // -LSE2 / c of each row (LSE2 in log2 units; -inf for padding rows: P = 0)
  float delta[QT];  // -Delta of each row
  int end[QT];      // prefix end e_b of the row (keys at or past it are masked)
};

__global__ __launch_bounds__(KV_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kv_kernel(BwdArgs a) {
  // Query tiles in the swizzled 320-byte layout: read row-major by the S and
  // dP products and transposed by the dV and dK products.
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][QT * LDS_ROW_SW];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2][QT * LDS_ROW_SW];
  __shared__ __attribute__((aligned(16))) QTileMeta sMeta[2];
  __shared__ __attribute__((aligned(16))) uint16_t sK[KV_KEYS * LDS_ROW];
  __shared__ int s_claim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);  // readfirstlane: the compiler keeps wave-level control flow scalar
  const int l32 = lane & 31, hf = lane >> 5;
  const SwizzledOffsets so = swizzled_offsets(lane);
  const int st_off = swizzled_store_off(tid);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  uint16_t* dK = static_cast<uint16_t*>(a.dk);
  uint16_t* dV = static_cast<uint16_t*>(a.dv);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;
  const float inv_c = 1.f / c;
  const int kv_st = (int)a.kv_st;  // a sequence's K/V span fits 31 bits of bytes (checked on the host)

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
      // in the packed copies, through buffer descriptors based at the tile's
      // first packed row (scalar work) with fixed 32-bit per-lane offsets.
      // Rows past the suffix (padding of the last tile) read as zeros, and
      // their LSE is set to +inf below, so they are masked.
      const int64_t vis0 = pbase + (int64_t)b_first * GB;  // packed index of the suffix's first row
      const int tq = wave * 64 + fresh_lane_id();
      const int qo = (tq >> 4) * (D * 2) + (tq & 15) * 16, mo = (tq & (QT - 1)) * 4;
      auto load_q = [&](int qt) {
        QTileRegs r;
        const int rows = min(nq - qt * QT, QT);
        const int64_t row0 = vis0 + qt * QT;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.qp + row0 * D, rows * D * 2);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.dop + row0 * D, rows * D * 2);
        r.q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 0));
        r.o = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ro, qo, 0, 0));
        // every thread loads a row's LSE, Delta and end (only threads 0..31
        // store them), so the loads issue with the tile's without a branch
        const float lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.lsep + row0, rows * 4), mo, 0, 0));
        const float del = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.deltap + row0, rows * 4), mo, 0, 0));
        const int e = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.endp + row0, rows * 4), mo, 0, 0);
        const bool in = (tid & (QT - 1)) < rows;
        r.lse = in ? lse : INFINITY;
        r.delta = in ? del : 0.f;
        r.end = in ? e : kb;
        return r;
      };
      auto store_q = [&](const QTileRegs& r, int buf) {
        *reinterpret_cast<uint4*>(sQ[buf] + st_off) = r.q;
        *reinterpret_cast<uint4*>(sdO[buf] + st_off) = r.o;
        if (tid < QT) {
          sMeta[buf].lse[tid] = -r.lse * inv_c;  // the S accumulators start here
          sMeta[buf].delta[tid] = -r.delta;  // the dP accumulators start at -Delta
          sMeta[buf].end[tid] = r.end;
        }
      };

      // This wave's 32 keys as MFMA B operands (k = head dim).
      const int kw0 = kb + wave * 32;           // first key of this wave
      const int key_w = kw0 + l32;
      // The first query tile's loads go out first: its addresses need only
      // b_first, and it is the last thing the pass waits for.
      QTileRegs R;
      if (ntq > 0) R = load_q(0);
      // K and V of the pass's keys through buffer descriptors based at key kb:
      // 32-bit offsets, and keys past the context read as zeros (their
      // entries are masked and their dK, dV rows are not written).
      const int kv_bytes = (n_ctx - kb) * kv_st * 2;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kseq + (int64_t)kb * a.kv_st, kv_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vseq + (int64_t)kb * a.kv_st, kv_bytes);
      // per-lane offsets formed here and hidden from the compiler, which
      // otherwise hoists them out of the loop and keeps them in scratch
      const int tf = wave * 64 + fresh_lane_id();
      const int vo = (wave * 32 + (tf & 31)) * kv_st * 2 + ((tf >> 5) & 1) * 16;
      const int ko = (tf >> 4) * kv_st * 2 + (tf & 15) * 16;
      bf16x8 vreg[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        vreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + ks * 32, 0, 0));
      uint4 kst[8];
      // 256 keys x 16 chunks of 16 bytes: thread -> key tid/16 + 32 u, chunk tid % 16
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kst[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + u * 64 * kv_st, 0, 0));
      __syncthreads();  // every wave is done with the previous pass's K
#pragma unroll
      for (int u = 0; u < 8; ++u)
        *reinterpret_cast<uint4*>(sK + ((tid >> 4) + 32 * u) * LDS_ROW + (tid & 15) * 8) = kst[u];
      f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dk_acc[i] = dv_acc[i] = f32x16{};
      const bool wave_live = kw0 < kend;        // the wave owns at least one key of the item

      if (ntq > 0) {
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
          uint32_t qt0 = lds_addr(bq + so.tr_off[0]), qt1 = lds_addr(bq + so.tr_off[1]);
          uint32_t ot0 = lds_addr(bo + so.tr_off[0]), ot1 = lds_addr(bo + so.tr_off[1]);
          asm volatile("" : "+v"(qt0), "+v"(qt1), "+v"(ot0), "+v"(ot1));

          // ---- S = Q K^T and dP = dO V^T for 32 rows x this wave's 32 keys ----
          // Two single chains (S, then dP), each with its LDS operands read one
          // k step ahead; interleaved, the compiler sank the reads back next to
          // their MFMAs and every step waited out a full LDS round trip.
          f32x16 sacc, pacc = f32x16{};
          const uint16_t* kw_ = sK + (wave * 32 + l32) * LDS_ROW + hf * 8;
          {
            // S - LSE2/c: the accumulators start at -LSE2/c of their rows
            // (element 4i + j: row 8i + 4hf + j), so P = exp2(c * acc)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 nl4 = *reinterpret_cast<const f32x4*>(&M.lse[8 * i + 4 * hf]);
#pragma unroll
              for (int j = 0; j < 4; ++j) sacc[4 * i + j] = nl4[j];
            }
            bf16x8 qa = lds_load_bf16x8(bq + so.row_off[0]);
            bf16x8 kf = lds_load_bf16x8(kw_);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              bf16x8 qn = qa, kn = kf;
              if (ks + 1 < 8) {
                const int ro = so.row_off[(ks + 1) & 1] + ((ks + 1) & ~1) * 16;
                qn = lds_load_bf16x8(bq + ro);
                kn = lds_load_bf16x8(kw_ + (ks + 1) * 16);
              }
              sacc = mfma32x32x16(qa, kf, sacc);
              asm volatile("" ::: "memory");
              qa = qn; kf = kn;
            }
          }
          {
            // dP - Delta: the accumulators start at -Delta of their rows
            // (element 4i + j: row 8i + 4hf + j).  P = exp2(c * acc) is taken
            // in place in the S accumulators, two entries per dP step, so the
            // exponentials issue while the dP products run.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 nd4 = *reinterpret_cast<const f32x4*>(&M.delta[8 * i + 4 * hf]);
#pragma unroll
              for (int j = 0; j < 4; ++j) pacc[4 * i + j] = nd4[j];
            }
            bf16x8 oa = lds_load_bf16x8(bo + so.row_off[0]);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              bf16x8 on = oa;
              if (ks + 1 < 8) on = lds_load_bf16x8(bo + so.row_off[(ks + 1) & 1] + ((ks + 1) & ~1) * 16);
              pacc = mfma32x32x16(oa, vreg[ks], pacc);
              sacc[2 * ks] = fast_exp2(sacc[2 * ks] * c);  // sacc holds s - LSE2/c
              sacc[2 * ks + 1] = fast_exp2(sacc[2 * ks + 1] * c);
              asm volatile("" ::: "memory");
              oa = on;
            }
          }
          // ---- P = 0 on masked entries, dS = P (dP - Delta) ----
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
                if (key_w >= ends[j]) sacc[4 * i + j] = 0.f;
            }
          }
          // ---- dV^T += dO^T P, dK^T += Q^T dS (A transposed from LDS, B = P, dS from registers) ----
          // P and dS of rows 0-15 first; those of rows 16-31 are formed a pair
          // at a time between the first half's products.  The transposed
          // operands of each product pair are read one pair ahead.
          uint32_t pk[2][4], dk2[2][4];
          auto form = [&](int kstep, int u) {  // entries 8 kstep + 2u, +1
            const int e = 8 * kstep + 2 * u;
            pk[kstep][u] = pack_bf16x2(sacc[e], sacc[e + 1]);
            dk2[kstep][u] = pack_bf16x2(sacc[e] * pacc[e], sacc[e + 1] * pacc[e + 1]);
          };
#pragma unroll
          for (int u = 0; u < 4; ++u) form(0, u);
          auto trq = [&](int kstep, int nd) { const uint32_t to = 2u * (kstep * 16 * LDS_ROW_SW + nd * 32); return lds_tr_pair(qt0 + to, qt1 + to); };
          auto tro = [&](int kstep, int nd) { const uint32_t to = 2u * (kstep * 16 * LDS_ROW_SW + nd * 32); return lds_tr_pair(ot0 + to, ot1 + to); };
          bf16x8 ob = tro(0, 0), qb = trq(0, 0);
#pragma unroll
          for (int kstep = 0; kstep < 2; ++kstep) {
            const bf16x8 pa = __builtin_bit_cast(bf16x8, uint4{pk[kstep][0], pk[kstep][1], pk[kstep][2], pk[kstep][3]});
            const bf16x8 da = __builtin_bit_cast(bf16x8, uint4{dk2[kstep][0], dk2[kstep][1], dk2[kstep][2], dk2[kstep][3]});
#pragma unroll
            for (int nd = 0; nd < 4; ++nd) {
              bf16x8 obn = ob, qbn = qb;
              if (kstep * 4 + nd + 1 < 8) {
                const int k2 = (kstep * 4 + nd + 1) >> 2, n2 = (nd + 1) & 3;
                obn = tro(k2, n2);
                qbn = trq(k2, n2);
              }
              dv_acc[nd] = mfma32x32x16(ob, pa, dv_acc[nd]);  // dV^T: head dim x keys
              dk_acc[nd] = mfma32x32x16(qb, da, dk_acc[nd]);  // dK^T
              if (kstep == 0) form(1, nd);
              asm volatile("" ::: "memory");
              ob = obn; qb = qbn;
            }
          }
        }
      }

      // ---- write dK (scaled) and dV for this wave's keys inside the item ----
      // The accumulators hold dK^T and dV^T: lane (l32, hf) has key key_w and
      // head dim nd*32 + 8r + 4hf + j in element 4r + j.  Swapping the 8-byte
      // runs of r = 2s+1 in the low lane half with those of r = 2s in the high
      // half gives each lane 16 consecutive bytes, head dim nd*32 + 16s + 8hf
      // onwards, so every store is 16 bytes.
      {
        const int64_t row = (k0 + key_w) * a.kv_st + (int64_t)g * a.kv_sh + 8 * hf;
        const bool own_key = key_w < kend;
#pragma unroll
        for (int nd = 0; nd < 4; ++nd)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const f32x16& ka = dk_acc[nd];
            const f32x16& va = dv_acc[nd];
            const int e0 = 8 * s2;
            const float sc = a.sm_scale;
            uint4 k4 = __builtin_bit_cast(uint4, to_bf16x8(sc * ka[e0], sc * ka[e0 + 1], sc * ka[e0 + 2], sc * ka[e0 + 3],
                                                         sc * ka[e0 + 4], sc * ka[e0 + 5], sc * ka[e0 + 6],
                                                         sc * ka[e0 + 7]));
            uint4 v4 = __builtin_bit_cast(uint4, to_bf16x8(va[e0], va[e0 + 1], va[e0 + 2], va[e0 + 3], va[e0 + 4],
                                                         va[e0 + 5], va[e0 + 6], va[e0 + 7]));
            swap_lane_halves(k4.x, k4.z);
            swap_lane_halves(k4.y, k4.w);
            swap_lane_halves(v4.x, v4.z);
            swap_lane_halves(v4.y, v4.w);
            if (own_key) {
              *reinterpret_cast<uint4*>(dK + row + nd * 32 + 16 * s2) = k4;
              *reinterpret_cast<uint4*>(dV + row + nd * 32 + 16 * s2) = v4;
            }
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
constexpr int DQ_WAVES = 8;             // two per SIMD
constexpr int DQ_THREADS = 64 * DQ_WAVES;
constexpr int DQ_ROWS = 32 * DQ_WAVES;  // packed query rows per pass
constexpr int DQ_NBUF = 3;
// K and V tiles of the query-owner kernel in the swizzled 320-byte layout
// (row-major K and V operands, transposed K operand).
constexpr int LDS_ROW_KV = LDS_ROW_SW;
constexpr int TILE_ELEMS = KT2 * LDS_ROW_KV;

// Staging registers of one K/V tile: rows tid/16 and tid/16 + 32, 16 bytes at
// head-dim 8*(tid%16), of K and of V.
struct KVTileRegs {
  uint4 k0, k1, v0, v1;
};

// Loads of key tile [kb, kb+64) through buffer descriptors based at key kb
// whose range ends with the context: keys past it read as zeros (they are
// masked for every row).
__device__ __forceinline__ KVTileRegs load_kv_tile(const uint16_t* Kseq, const uint16_t* Vseq, int kb, int n_ctx,
                                                   int kv_st, int o0) {
  const int64_t start = (int64_t)kb * kv_st;
  const int range = (n_ctx - kb) * kv_st * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kseq + start, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vseq + start, range);
  const int o1 = o0 + 32 * kv_st * 2;
  KVTileRegs r;
  r.k0 = buffer_load_b128(rk, o0);
  r.k1 = buffer_load_b128(rk, o1);
  r.v0 = buffer_load_b128(rv, o0);
  r.v1 = buffer_load_b128(rv, o1);
  return r;
}

__device__ __forceinline__ void store_kv_tile(const KVTileRegs& r, uint16_t* sK, uint16_t* sV, int tid) {
  const int o = swizzled_store_off(tid);
  constexpr int R32 = 32 * LDS_ROW_KV;
  *reinterpret_cast<uint4*>(sK + o) = r.k0;
  *reinterpret_cast<uint4*>(sK + o + R32) = r.k1;
  *reinterpret_cast<uint4*>(sV + o) = r.v0;
  *reinterpret_cast<uint4*>(sV + o + R32) = r.v1;
}

__global__ __launch_bounds__(DQ_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  // Three K/V buffers: tile t+1 is stored while tile t is computed, tile t+2
  // is in flight, so one barrier per tile suffices (as in the forward).
  __shared__ __attribute__((aligned(16))) uint16_t sKV[DQ_NBUF][2][TILE_ELEMS];
  __shared__ int s_claim;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;
  const int kv_st = (int)a.kv_st;  // a sequence's K/V span fits 31 bits of bytes (checked on the host)
  const int ld_off = (tid >> 4) * kv_st * 2 + (tid & 15) * 16;
  // swizzled element offsets of this lane's row-major and transposed reads
  int kv_row_off[2], kt_off[2];
  {
    const int gi = lane >> 4, li = lane & 15;
    const int f = (l32 >> 2) & 3;
#pragma unroll
    for (int k = 0; k < 2; ++k) kv_row_off[k] = l32 * LDS_ROW_KV + 16 * (k ^ (f >> 1)) + 8 * (hf ^ (f & 1));
    const int c1 = (2 * (gi & 1) + ((li & 3) >> 1)) ^ hf;
    kt_off[0] = (4 * hf + (li >> 2)) * LDS_ROW_KV + 8 * c1 + 4 * (li & 1);
    kt_off[1] = (4 * hf + (li >> 2) + 8) * LDS_ROW_KV + 8 * (c1 ^ 2) + 4 * (li & 1);
  }

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
    for (int rt = 0; rt < nrows; rt += DQ_ROWS) {
      const int p_last = min(nrows, rt + DQ_ROWS) - 1;
      const int wg_hi = max(klo, min(khi, a.endp[pitem + p_last]));
      const int ntiles = (wg_hi - klo + KT2 - 1) / KT2;
      if (ntiles == 0) continue;  // no row of the pass sees the chunk: no partial to write

      __syncthreads();  // all waves are done with the previous pass's buffers
      KVTileRegs R = load_kv_tile(Kseq, Vseq, klo, n_ctx, kv_st, ld_off);
      // ---- this lane's row: Q and dO as MFMA B operands, LSE, Delta ----
      const int p = rt + wave * 32 + l32;
      const bool valid = p < nrows;
      const int pc = valid ? p : p_last;  // clamp: loads stay in bounds, results unused
      const int b = it.lo + a.fd_gb.div(pc);
      const int hl = a.fd_group.mod(a.fd_block.div(pc));
      const int64_t r = (int64_t)b * a.block + a.fd_block.mod(pc);
      const int h = it.kv_head * a.group + hl;
      const int64_t P = pitem + pc;
      const int e = a.endp[P];
      const int vend = valid ? max(klo, min(khi, e)) : klo;  // visible keys of the row: [klo, vend)
      const int64_t prow = part_base + (int64_t)h * mq + r;
      const float lse2 = a.lsep[P];
      const float del = a.deltap[P];
      bf16x8 qf[8], of[8];
      {
        const uint16_t* qrow = a.qp + P * D + hf * 8;
        const uint16_t* orow = a.dop + P * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          qf[ks] = load_bf16x8(qrow + ks * 16);
          of[ks] = load_bf16x8(orow + ks * 16);
        }
      }
      store_kv_tile(R, sKV[0][0], sKV[0][1], tid);
      // Drain every outstanding load before the prefetch starts, so that
      // inside the tile loop only the prefetch itself is in flight.
      __builtin_amdgcn_s_waitcnt(0);
      if (ntiles > 1) R = load_kv_tile(Kseq, Vseq, klo + KT2, n_ctx, kv_st, ld_off);
      const int wave_hi = wave_max_i(vend);
      const int wave_full = wave_min_i(valid ? vend : INT32_MAX);

      f32x16 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

      for (int t = 0; t < ntiles; ++t) {
        const int kb = klo + t * KT2;
        __syncthreads();  // tile t, stored during tile t-1, is visible
        // Tile t+1 goes into the buffer tile t-2 used (free since the
        // previous barrier), after this barrier, so that the barrier does not
        // wait for these stores; the next one finds them complete.
        if (t + 1 < ntiles) {
          store_kv_tile(R, sKV[(t + 1) % DQ_NBUF][0], sKV[(t + 1) % DQ_NBUF][1], tid);
          if (t + 2 < ntiles) R = load_kv_tile(Kseq, Vseq, kb + 2 * KT2, n_ctx, kv_st, ld_off);
        }
        if (kb >= wave_hi) continue;  // no row of this wave sees the tile (nor any later one)
        // 32-bit LDS addresses of this lane's reads in the tile's buffers; the
        // empty asm keeps every per-read offset an immediate instead of one
        // address add per read.
        uint32_t ka[2], va[2], kt[2];
        {
          const uint32_t kb_ = lds_addr(sKV[t % DQ_NBUF][0]), vb_ = lds_addr(sKV[t % DQ_NBUF][1]);
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            ka[k] = kb_ + 2u * kv_row_off[k];
            va[k] = vb_ + 2u * kv_row_off[k];
            kt[k] = kb_ + 2u * kt_off[k];
          }
          asm volatile("" : "+v"(ka[0]), "+v"(ka[1]), "+v"(va[0]), "+v"(va[1]), "+v"(kt[0]), "+v"(kt[1]));
        }

        // Per 32-key half mt: S^T = K Q^T and dP^T = V dO^T (A from LDS),
        // dS^T = P^T (dP^T - Delta) with P^T = exp2(s*c - LSE2) on visible keys,
        // then dQ^T += K^T dS^T (K^T read transposed from LDS).
        auto tile = [&](auto mask_c) {
          constexpr bool MASK = decltype(mask_c)::value;  // partial tile: keys past a row's end are masked
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const uint32_t mo = 2u * (mt * 32 * LDS_ROW_KV);  // byte offset of the half's rows
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            {  // S^T chain, operands read one k step ahead
              bf16x8 kf = lds_read_b128(ka[0] + mo);
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                bf16x8 kn = kf;
                if (ks + 1 < 8) kn = lds_read_b128(ka[(ks + 1) & 1] + mo + 2u * (((ks + 1) & ~1) * 16));
                sacc = mfma32x32x16(kf, qf[ks], sacc);
                asm volatile("" ::: "memory");
                kf = kn;
              }
            }
            {  // dP^T - Delta chain: the accumulator starts at -Delta of this lane's row
#pragma unroll
              for (int e2 = 0; e2 < 16; ++e2) pacc[e2] = -del;
              bf16x8 vf = lds_read_b128(va[0] + mo);
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                bf16x8 vn = vf;
                if (ks + 1 < 8) vn = lds_read_b128(va[(ks + 1) & 1] + mo + 2u * (((ks + 1) & ~1) * 16));
                pacc = mfma32x32x16(vf, of[ks], pacc);
                asm volatile("" ::: "memory");
                vf = vn;
              }
            }
            // element e holds key kb + mt*32 + 8*(e/4) + 4*hf + e%4 of this lane's row
            const int lim = vend - kb - mt * 32 - hf * 4;  // keys at or past the row's end are masked
#pragma unroll
            for (int e2 = 0; e2 < 16; ++e2) {
              float pe = fast_exp2(__builtin_fmaf(sacc[e2], c, -lse2));
              if (MASK && (e2 >> 2) * 8 + (e2 & 3) >= lim) pe = 0.f;
              sacc[e2] = pe * pacc[e2];  // pacc holds dP - Delta
            }
            // dQ^T += K^T dS^T, the K^T operand read one step ahead
            const bf16x8 df0 = to_bf16x8(sacc[0], sacc[1], sacc[2], sacc[3], sacc[4], sacc[5], sacc[6], sacc[7]);
            const bf16x8 df1 = to_bf16x8(sacc[8], sacc[9], sacc[10], sacc[11], sacc[12], sacc[13], sacc[14], sacc[15]);
            bf16x8 ktc = lds_tr_pair(kt[0] + 2u * (2 * mt * 16 * LDS_ROW_KV), kt[1] + 2u * (2 * mt * 16 * LDS_ROW_KV));
#pragma unroll
            for (int st = 0; st < 8; ++st) {  // st = half * 4 + md
              bf16x8 ktn = ktc;
              if (st + 1 < 8) {
                const int o = (2 * mt + ((st + 1) >> 2)) * 16 * LDS_ROW_KV + ((st + 1) & 3) * 32;
                ktn = lds_tr_pair(kt[0] + 2u * o, kt[1] + 2u * o);
              }
              acc[st & 3] = mfma32x32x16(ktc, (st >> 2) ? df1 : df0, acc[st & 3]);
              asm volatile("" ::: "memory");
              ktc = ktn;
            }
          }
        };
        if (kb + KT2 > wave_full) tile(std::integral_constant<bool, true>{});
        else tile(std::integral_constant<bool, false>{});
      }

      // ---- the item's dQ partial (unscaled) for a row that sees its keys ----
      if (valid && vend > klo) {
        if (hf == 0) a.dq_run[prow] = n_chunk;
        float* op = a.dq_part + prow * D + hf * 4;
#pragma unroll
        for (int md = 0; md < 4; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 v4 = {acc[md][4 * i + 0], acc[md][4 * i + 1], acc[md][4 * i + 2], acc[md][4 * i + 3]};
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
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(q_workers), dim3(DQ_THREADS), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess || rows == 0) return e;
  }
  if (a.own && (e = launch_own_bwd(a, a.total_q / a.block, stream)) != hipSuccess) return e;
  TimedLaunch t(kBwdFinalize, stream);
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
