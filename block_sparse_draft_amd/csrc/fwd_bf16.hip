// Split-KV partial forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// The contribution of one KV chunk, or of a run of consecutive chunks, to the
// attention of a range of draft blocks (pages: Split-KV article, "Split-KV's
// Core Mechanism": each KV shard stays local and yields a query-sized result
// that is later aggregated exactly).
//
// Persistent workgroups of 8 waves (two per SIMD, so one wave's softmax and
// memory waits overlap the other's MFMA work): each runs the work items the
// planner gave its worker, then claims whatever is left on other workers'
// lists.  An item is (sequence, KV head g with its G query heads, chunks
// c .. c + n_chunk - 1, draft blocks [lo, hi)); it writes one partial, in
// chunk c's rows.  Its query rows are packed block-major as
// p = ((b - lo) * G + head) * B + token, 256 rows per pass: 8 waves x 32 rows.
// Each wave keeps its 32 Q rows in registers and the unnormalised O^T
// (128 x 32, fp32) in accumulators.  Only the 64-key tiles that some row of
// the pass sees are visited; the rest of the chunk is never read.
//
// Pipeline: K/V tiles rotate through three LDS buffers.  While tile t is
// computed, tile t+1 sits in LDS and tile t+2 is in flight from memory into
// registers, so a single barrier per tile suffices.  K is staged row-major;
// V is staged transposed (V^T, one row per head-dim index), its keys permuted
// within each 16-key group to the order the PV product consumes them, so every
// MFMA operand read is one 16-byte LDS read.
//
// Per key tile and wave:  S^T = K Q^T (MFMA 32x32x16), masking of keys at or
// beyond the row's prefix end e_b (partial tiles only), online softmax in the
// exp2 domain with lazy rescaling (the reference maximum only moves when the
// true maximum exceeds it by 2^8; the output is corrected to the true maximum
// once per item), O^T += V^T P^T with P^T taken straight from the S^T
// accumulators.  Each tile's scores are computed right before its softmax:
// the wave's own MFMA latency is covered by the other wave of its SIMD, and a
// cross-tile pipeline (the scores of tile t+1 before the softmax of tile t)
// measured 4% slower, for its second set of score registers and their copies.
// Every LDS operand is read one MFMA step ahead of its use, and K/V tiles are
// fetched through buffer descriptors so that the per-tile address work is
// scalar.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int D = 128;
constexpr int KT = 64;              // keys per tile
constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int ROWS = 32 * NWAVE;    // packed query rows per pass
constexpr int NBUF = 3;
constexpr float LAZY_LOG2 = 8.f;    // rescale only when the max grows by more than 2^8
// Padded LDS rows: 272-byte K rows put the 16-byte operand reads of 16
// consecutive rows in distinct banks.  V^T rows are 192 bytes with their eight
// 16-byte key chunks XOR-swizzled by bits 2..4 of the row (chunk c of row r
// sits at c ^ ((r >> 2) & 7)): measured with the LDS bank-conflict counter,
// both the 8-byte staging writes and the 16-byte operand reads then run at
// their conflict-free rate (a 144-byte unswizzled layout serialises the
// writes 8 ways).
constexpr int LDS_ROW_K = D + 8;
constexpr int LDS_ROW_VT = KT + 32;
constexpr int TILE_K = KT * LDS_ROW_K;
constexpr int TILE_VT = D * LDS_ROW_VT;

// Staging registers of one K/V tile.  K: 2 x 16 bytes (rows r and r + 32,
// 8 head-dim values each).  V: 4 keys x 4 head-dim values (8 bytes per key).
// V key groups (4 keys each): wave w stages groups g0 = 4 (w / 2) + w % 2 and
// g0 + 2 (even and odd lanes), head-dim values 4 (lane / 2) .. + 3.
struct TileRegs {
  uint4 k0, k1;
  uint2 v0, v1, v2, v3;
};

__device__ __forceinline__ int v_group(int tid) {
  const int w = tid >> 6;
  return 4 * (w >> 1) + (w & 1) + 2 * (tid & 1);
}

// Byte offsets of this thread's staging loads inside a tile: K rows tid/16 and
// tid/16 + 32 (16 bytes at head-dim 8*(tid%16)); V keys 4*g + j of its key
// group g (8 bytes at head-dim 4*((tid%64)/2)).
struct TileOffsets {
  int k0, k1, v0, v1, v2, v3;
};

__device__ __forceinline__ TileOffsets tile_offsets(int kv_st, int tid) {
  TileOffsets o;
  const int rb = kv_st * 2;  // bytes per key row
  o.k0 = (tid >> 4) * rb + (tid & 15) * 16;
  o.k1 = o.k0 + 32 * rb;
  o.v0 = v_group(tid) * 4 * rb + ((tid & 63) >> 1) * 8;
  o.v1 = o.v0 + rb;
  o.v2 = o.v0 + 2 * rb;
  o.v3 = o.v0 + 3 * rb;
  return o;
}

// Issue the loads of key tile [kb, kb+64) (sequence-relative) through buffer
// descriptors based at key kb whose range ends with the context: keys past
// the context read as zeros (they are masked for every row).  The per-tile
// address work is scalar and each thread keeps six 32-bit offsets.
__device__ __forceinline__ TileRegs load_tile(const uint16_t* Kseq, const uint16_t* Vseq, int kb, int n_ctx,
                                              int kv_st, const TileOffsets& o) {
  const int64_t start = (int64_t)kb * kv_st;
  const int range = (n_ctx - kb) * kv_st * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kseq + start, range);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vseq + start, range);
  TileRegs r;
  r.k0 = buffer_load_b128(rk, o.k0);
  r.k1 = buffer_load_b128(rk, o.k1);
  r.v0 = buffer_load_b64(rv, o.v0);
  r.v1 = buffer_load_b64(rv, o.v1);
  r.v2 = buffer_load_b64(rv, o.v2);
  r.v3 = buffer_load_b64(rv, o.v3);
  return r;
}

// Position of key kk (0..15) of a 16-key group inside a V^T row (before the
// swizzle): lane half h of the PV operand reads positions 8h..8h+7, which hold
// keys 4h..4h+3 and 8+4h..8+4h+3 (the order the S^T accumulators deliver P^T
// in).  Key group g (keys 4g..4g+3) thus fills 16-byte chunk 2 (g / 4) + g % 2,
// 8-byte half (g / 2) % 2.
__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* sK, uint16_t* sVt, int tid) {
  *reinterpret_cast<uint4*>(sK + (tid >> 4) * LDS_ROW_K + (tid & 15) * 8) = r.k0;
  *reinterpret_cast<uint4*>(sK + ((tid >> 4) + 32) * LDS_ROW_K + (tid & 15) * 8) = r.k1;
  // 4 keys x 4 values -> 4 rows of V^T with 4 keys each
  const int kg = v_group(tid);                              // keys 4kg .. 4kg+3
  const int h4 = (tid & 63) >> 1;                           // V^T rows 4h4 .. 4h4+3
  const int chunk = (2 * (kg >> 2) + (kg & 1)) ^ (h4 & 7);  // rows 4h4 + j share the swizzle
  uint16_t* dst = sVt + h4 * 4 * LDS_ROW_VT + chunk * 8 + ((kg >> 1) & 1) * 4;
  // byte selectors of v_perm_b32(hi, lo, sel): bytes 0-3 from lo, 4-7 from hi
  const uint32_t lo16 = 0x05040100u, hi16 = 0x07060302u;
  uint2 y0, y1, y2, y3;
  y0.x = __builtin_amdgcn_perm(r.v1.x, r.v0.x, lo16); y0.y = __builtin_amdgcn_perm(r.v3.x, r.v2.x, lo16);
  y1.x = __builtin_amdgcn_perm(r.v1.x, r.v0.x, hi16); y1.y = __builtin_amdgcn_perm(r.v3.x, r.v2.x, hi16);
  y2.x = __builtin_amdgcn_perm(r.v1.y, r.v0.y, lo16); y2.y = __builtin_amdgcn_perm(r.v3.y, r.v2.y, lo16);
  y3.x = __builtin_amdgcn_perm(r.v1.y, r.v0.y, hi16); y3.y = __builtin_amdgcn_perm(r.v3.y, r.v2.y, hi16);
  *reinterpret_cast<uint2*>(dst) = y0;
  *reinterpret_cast<uint2*>(dst + LDS_ROW_VT) = y1;
  *reinterpret_cast<uint2*>(dst + 2 * LDS_ROW_VT) = y2;
  *reinterpret_cast<uint2*>(dst + 3 * LDS_ROW_VT) = y3;
}

__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sKb[NBUF][TILE_K];
  __shared__ __attribute__((aligned(16))) uint16_t sVb[NBUF][TILE_VT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const int GB = a.group * a.block;
  const float c = a.scale_log2;
  const int kv_st = (int)a.kv_st;  // the host checks that a sequence's K/V span fits 31 bits of bytes
  const TileOffsets toff = tile_offsets(kv_st, tid);
  const uint32_t va_lane = 2u * (l32 * LDS_ROW_VT) + 16u * (hf ^ ((l32 >> 2) & 1));
  const int va_z = (l32 >> 3) & 3;

  __shared__ int s_claim;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int me = plan_worker();
  int victim = me, visited = 0;
  for (;;) {
    const int64_t slot = claim_next(a.worker_off, a.claim, victim, visited, &s_claim, a.steal);
    if (slot < 0) break;
    skv_item it = a.items[slot];
    it.seq = uniform(it.seq); it.kv_head = uniform(it.kv_head); it.chunk = uniform(it.chunk);
    it.lo = uniform(it.lo); it.hi = uniform(it.hi); it.part_base = uniform(it.part_base);
    it.n_chunk = uniform(it.n_chunk);
    const int s = it.seq;
    const int64_t q0 = uniform(a.q_off[s]);
    const int64_t mq = uniform(a.q_off[s + 1]) - q0;
    const int64_t k0 = uniform(a.kv_off[s]);
    const int n_ctx = (int)(uniform(a.kv_off[s + 1]) - k0);
    const int64_t blk0 = q0 / a.block;
    // keys of the item's chunks: [chunk*L, (chunk + n_chunk)*L) inside the context
    const int klo = it.chunk * a.chunk;
    const int khi = (int)min((int64_t)(it.chunk + max(1, it.n_chunk)) * a.chunk, (int64_t)n_ctx);
    const int nrows = (it.hi - it.lo) * GB;
    const uint16_t* Kseq = K + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;
    const uint16_t* Vseq = V + k0 * a.kv_st + (int64_t)it.kv_head * a.kv_sh;

    for (int rt = 0; rt < nrows; rt += ROWS) {
      // Anchors are sorted, so the last row of the pass has the largest prefix end.
      const int p_last = min(nrows, rt + ROWS) - 1;
      const int wg_hi = max(klo, min(khi, min(a.anchor[blk0 + it.lo + a.fd_gb.div(p_last)] + a.end_shift, n_ctx)));
      const int ntiles = (wg_hi - klo + KT - 1) / KT;

      // ---- start the K/V pipeline around the loads of this lane's Q row ----
      TileRegs R;
      if (ntiles > 0) {
        __syncthreads();  // all waves are done with the previous pass's buffers
        R = load_tile(Kseq, Vseq, klo, n_ctx, kv_st, toff);
      }
      const int p = rt + wave * 32 + l32;
      const bool valid = p < nrows;
      const int pc = valid ? p : p_last;  // clamp: loads stay in bounds, results unused
      const int b = it.lo + a.fd_gb.div(pc);
      const int hl = a.fd_group.mod(a.fd_block.div(pc));
      const int64_t r = (int64_t)b * a.block + a.fd_block.mod(pc);
      const int h = it.kv_head * a.group + hl;
      const int e = min(a.anchor[blk0 + b] + a.end_shift, n_ctx);
      const int vend = valid ? max(klo, min(khi, e)) : klo;  // visible keys of the row: [klo, vend)
      const int64_t prow = it.part_base + (int64_t)h * mq + r;
      bf16x8 qf[8];
      {
        const uint16_t* qp = Q + (q0 + r) * a.q_st + (int64_t)h * a.q_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = load_bf16x8(qp + ks * 16);
      }
      if (ntiles > 0) store_tile(R, sKb[0], sVb[0], tid);
      // Drain every outstanding load (Q included) before the prefetch starts, so
      // that inside the tile loop only the prefetch itself is in flight.
      __builtin_amdgcn_s_waitcnt(0);
      if (ntiles > 1) R = load_tile(Kseq, Vseq, klo + KT, n_ctx, kv_st, toff);
      const int wave_hi = wave_max_i(vend);
      const int wave_full = wave_min_i(valid ? vend : INT32_MAX);

      float m_true = -INFINITY;  // running row max of raw scores
      float m_ref = -INFINITY;   // max the exponentials are taken against
      float l = 0.f;             // this lane-half's running row sum
      f32x16 acc_o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};

      // S^T = K Q^T of the tile in buffer `buf` (raw scores), 16 MFMAs.  The K
      // operands of k step ks+1 are read before the MFMAs of k step ks, so a
      // read's latency overlaps the previous step's products.
      auto scores = [&](int buf, f32x16 (&sacc)[2]) {
        uint32_t ka = lds_addr(sKb[buf] + l32 * LDS_ROW_K + hf * 8);
        asm volatile("" : "+v"(ka));  // keeps the per-read offsets as immediates
        sacc[0] = sacc[1] = f32x16{};
        bf16x8 kc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) kc[mt] = lds_read_b128(ka + 2u * (mt * 32 * LDS_ROW_K));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          bf16x8 kn[2] = {kc[0], kc[1]};
          if (ks + 1 < 8) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) kn[mt] = lds_read_b128(ka + 2u * (mt * 32 * LDS_ROW_K + (ks + 1) * 16));
          }
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma32x32x16(kc[mt], qf[ks], sacc[mt]);
          kc[0] = kn[0];
          kc[1] = kn[1];
        }
      };

      f32x16 scur[2];  // this tile's scores S^T
      for (int t = 0; t < ntiles; ++t) {
        const int kb = klo + t * KT;
        if (t + 1 < ntiles) {
          store_tile(R, sKb[(t + 1) % NBUF], sVb[(t + 1) % NBUF], tid);
          if (t + 2 < ntiles) R = load_tile(Kseq, Vseq, kb + 2 * KT, n_ctx, kv_st, toff);
        }
        __syncthreads();
        if (kb >= wave_hi) continue;  // no row of this wave sees the tile (nor any later one)
        scores(t % NBUF, scur);

        // ---- mask keys at or past the row's prefix end (partial tiles only) ----
        if (kb + KT > wave_full) {
          // element e2 of half mt holds key kb + mt*32 + 8*(e2/4) + 4*hf + e2%4
          const int lim = vend - kb - 4 * hf;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e2 = 0; e2 < 16; ++e2)
              if (mt * 32 + (e2 >> 2) * 8 + (e2 & 3) >= lim) scur[mt][e2] = -INFINITY;
        }
        // ---- row max; lazy rescale when the row's max grew past 2^8 ----
        // two v_max3 chains (one per 32-key half), two new scores per instruction
        float r0 = fmaxf(scur[0][0], scur[0][1]), r1 = fmaxf(scur[1][0], scur[1][1]);
#pragma unroll
        for (int e2 = 2; e2 < 16; e2 += 2) {
          r0 = max3f(r0, scur[0][e2], scur[0][e2 + 1]);
          r1 = max3f(r1, scur[1][e2], scur[1][e2 + 1]);
        }
        r0 = max_lane_halves(fmaxf(r0, r1));
        m_true = fmaxf(m_true, r0);
        const bool grow = (m_true - m_ref) * c > LAZY_LOG2;  // false while both are -inf
        if (__any(grow)) {
          const float alpha = fast_exp2((m_ref - m_true) * c);  // 0 from -inf, 1 if unchanged
          const bool keep = m_true == -INFINITY;
          m_ref = m_true;
          if (!keep) {
            l *= alpha;
#pragma unroll
            for (int md = 0; md < 4; ++md) acc_o[md] *= alpha;
          }
        }
        // ---- P = exp2(s*c - m_ref*c), 16 keys per step of O^T += V^T P^T;
        //      the row sum in fp32 (bf16-rounded P would cost the log-sum-exp
        //      up to 2^-9 relative on short rows).  The next step's
        //      exponentials are taken between this step's four MFMAs, so they
        //      issue while the products run, and its V operands are read
        //      before them; the empty asm ends each step's scheduling region,
        //      which bounds how many operands the compiler keeps in flight. ----
        // Row md*32 + l32, key chunk 2 kstep + hf, swizzle f = (l32 / 4) % 8:
        // this lane's chunk pair sits at 32-byte slot kstep ^ (f / 2), its
        // half at 16 (hf ^ f % 2), the same for every md.
        const uint32_t vrow = lds_addr(sVb[t % NBUF]) + va_lane;
        uint32_t va[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) va[k] = vrow + 32u * (k ^ va_z);
        asm volatile("" : "+v"(va[0]), "+v"(va[1]), "+v"(va[2]), "+v"(va[3]));
        auto vaddr = [&](int md, int ks) { return va[ks] + 2u * (md * 32 * LDS_ROW_VT); };
        const float mc = m_ref == -INFINITY ? 0.f : m_ref * c;
        // P of step kstep: entries 8 (kstep % 2) .. +7 of half kstep / 2, as
        // four bf16 pairs; the row sum adds them in a fixed tree.
        uint32_t pk[2][4];
        float ps[2][4];
        auto form = [&](int kstep, int u) {
          const f32x16& sv = scur[kstep >> 1];
          const int e = (kstep & 1) * 8 + 2 * u;
          const float p0 = fast_exp2(__builtin_fmaf(sv[e], c, -mc));
          const float p1 = fast_exp2(__builtin_fmaf(sv[e + 1], c, -mc));
          pk[kstep & 1][u] = pack_bf16x2(p0, p1);
          ps[kstep & 1][u] = p0 + p1;
        };
        bf16x8 vc[4];
#pragma unroll
        for (int md = 0; md < 4; ++md) vc[md] = lds_read_b128(vaddr(md, 0));
#pragma unroll
        for (int u = 0; u < 4; ++u) form(0, u);
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          const int b = kstep & 1;
          const bf16x8 pf = __builtin_bit_cast(bf16x8, uint4{pk[b][0], pk[b][1], pk[b][2], pk[b][3]});
          l += (ps[b][0] + ps[b][1]) + (ps[b][2] + ps[b][3]);
          bf16x8 vn[4] = {vc[0], vc[1], vc[2], vc[3]};
          if (kstep + 1 < 4) {
#pragma unroll
            for (int md = 0; md < 4; ++md) vn[md] = lds_read_b128(vaddr(md, kstep + 1));
          }
#pragma unroll
          for (int md = 0; md < 4; ++md) {
            acc_o[md] = mfma32x32x16(vc[md], pf, acc_o[md]);
            if (kstep + 1 < 4) form(kstep + 1, md);
          }
          asm volatile("" ::: "memory");
#pragma unroll
          for (int md = 0; md < 4; ++md) vc[md] = vn[md];
        }
      }

      // ---- epilogue: unnormalised O_c against the true row max, max and log-sum-exp ----
      float lt = sum_lane_halves(l);
      if (valid) {
        const bool seen = lt > 0.f;
        const float fix = seen ? fast_exp2((m_ref - m_true) * c) : 1.f;
        lt *= fix;
        if (hf == 0) {
          a.m_part[prow] = seen ? m_true * a.sm_scale : -INFINITY;
          a.lse_part[prow] = seen ? (m_true * c + __log2f(lt)) * kLn2 : -INFINITY;
        }
        if (seen) {
          float* op = a.o_part + prow * D + hf * 4;
#pragma unroll
          for (int md = 0; md < 4; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              f32x4 v4 = {acc_o[md][4 * i + 0] * fix, acc_o[md][4 * i + 1] * fix, acc_o[md][4 * i + 2] * fix,
                          acc_o[md][4 * i + 3] * fix};
              *reinterpret_cast<f32x4*>(op + md * 32 + 8 * i) = v4;
            }
        }
      }
    }
  }
  record_ticks(a.ticks, me, t_start);
}

// m = lse = -inf for every partial row (rows of items left out of a plan);
// the plan's claim cursors are reset in the same launch.
__global__ __launch_bounds__(256) void fill_neg_inf_kernel(float* m, float* lse, int64_t n, int32_t* claim,
                                                           int n_claim) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n_claim) claim[t] = 0;
  const int64_t i = t * 4;
  if (i >= n) return;
  const f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (i + 4 <= n && ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(lse)) & 15) == 0) {
    *reinterpret_cast<f32x4*>(m + i) = v;
    *reinterpret_cast<f32x4*>(lse + i) = v;
  } else {
    for (int64_t j = i; j < min(i + 4, n); ++j) m[j] = lse[j] = -INFINITY;
  }
}

}  // namespace


hipError_t launch_fill_neg_inf(float* m, float* lse, int64_t n, int32_t* claim, int n_claim, hipStream_t stream) {
  const int64_t blocks = std::max<int64_t>((n + 1023) / 1024, (n_claim + 255) / 256);
  if (blocks == 0) return hipSuccess;
  TimedLaunch t(kFillPartials, stream);
  hipLaunchKernelGGL(fill_neg_inf_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, m, lse, n, claim, n_claim);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int n_workers, hipStream_t stream) {
  TimedLaunch t(kFwdBf16, stream);
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(n_workers), dim3(NTHR), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
