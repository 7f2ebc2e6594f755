// Kernel argument blocks and launchers of libsplitkv (host <-> device glue).
// Launchers enqueue on `stream` and return hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"
#include "splitkv.h"

namespace skv {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_st, q_sh, kv_st, kv_sh;  // element strides
  const int64_t* q_off;
  const int64_t* kv_off;
  const int32_t* anchor;
  const skv_item* items;
  const int64_t* worker_off;
  int32_t* claim;
  int64_t* ticks;  // optional per-workgroup busy time
  int32_t steal;   // claim from other workers' lists once the own list is done
  float* o_part;
  float* m_part;
  float* lse_part;
  int32_t block, group, hq, chunk;
  int32_t end_shift;  // e_b = min(a_b + end_shift, N): block (prefix mask) or 0 (own-block mask)
  FastDiv fd_block, fd_group, fd_gb;  // division by block, hq/hkv and their product
  float sm_scale;
  float scale_log2;  // sm_scale * log2(e)
};

// Own-block partial (own-block mask): one workgroup per (draft block, KV head).
struct OwnFwdArgs {
  const void* q;
  const void* k_own;
  const void* v_own;
  int64_t q_st, q_sh, own_st, own_sh;  // element strides
  const int64_t* q_off;
  const int64_t* kv_off;
  float* o_part;
  float* m_part;
  float* lse_part;
  int32_t n_seq, block, group, hq, hkv, chunk;
  float sm_scale;
};

struct MergeArgs {
  const float* o_part;
  const float* m_part;
  const float* lse_part;
  void* o_out;
  float* lse_out;
  int64_t mq, o_st, o_sh, lse_st;  // mq: rows (all sequences' rows when n_seq > 0)
  int32_t n_part, hq, out_bf16;
  // n_seq > 0: rows of several sequences, row t of sequence s (q_off) with
  // its partials at part_base[s] + c*hq*Mq_s + h*Mq_s + (t - q_off[s]);
  // n_seq = 0: one sequence, n_part partials at c*hq*mq + h*mq + t.
  const int64_t* q_off;
  const int64_t* part_base;
  int32_t n_seq;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dq_part;     // dQ partials, the forward's partial layout, [rows][d] fp32
  int32_t* dq_run;    // [rows]: chunks covered by the dQ partial in that row (written with it)
  // Packed row order: row P = q_off[s]*hq + g*G*Mq_s + (b*G + hl)*B + i holds
  // token q_off[s] + b*B + i of query head g*G + hl.
  uint16_t* qp;       // [sum Mq * hq][d] bf16 copy of Q
  uint16_t* dop;      // [sum Mq * hq][d] bf16 copy of dO
  float* lsep;        // LSE * log2(e)
  float* deltap;      // Delta = sum_x dO * O
  int32_t* endp;      // prefix end e_b of the row's draft block
  int64_t* part_base; // [n_seq + 1] first partial row of each sequence
  int64_t q_st, q_sh, kv_st, kv_sh;
  const int64_t* q_off;
  const int64_t* kv_off;
  const int32_t* anchor;
  const skv_item* kv_items;      // BWD plan: key ranges
  const int64_t* kv_worker_off;
  int32_t* kv_claim;
  int64_t* kv_ticks;
  const skv_item* q_items;       // FWD plan: draft-block ranges of one chunk
  const int64_t* q_worker_off;
  int32_t* q_claim;
  int64_t* q_ticks;
  int32_t kv_steal, q_steal;
  int32_t kv_claim_n, q_claim_n;  // claim cursors reset by the first launch of the backward
  int64_t total_q;  // sum Mq
  int32_t n_seq, block, group, hq, hkv, chunk;
  int32_t end_shift;  // e_b = min(a_b + end_shift, N): block (prefix mask) or 0 (own-block mask)
  int32_t own;        // own-block mask: one more dQ partial per sequence (index C_s)
  const void* k_own;  // own-block keys / values and their gradients, [sum Mq][hkv][d]
  const void* v_own;
  void* dk_own;
  void* dv_own;
  int64_t own_st, own_sh;
  FastDiv fd_block, fd_group, fd_gb;  // division by block, hq/hkv and their product
  float sm_scale, scale_log2;
};

hipError_t launch_fill_neg_inf(float* m, float* lse, int64_t n, int32_t* claim, int n_claim, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, int n_workers, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, int n_workers, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, int kv_workers, int q_workers, hipStream_t stream);
hipError_t launch_own_fwd(const OwnFwdArgs& a, int dtype, int d, int64_t n_blocks, hipStream_t stream);
hipError_t launch_own_bwd(const BwdArgs& a, int64_t n_blocks, hipStream_t stream);

}  // namespace skv
