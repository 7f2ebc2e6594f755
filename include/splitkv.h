/*
 * splitkv.h — C ABI of libsplitkv: Split-KV block-sparse draft attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes (pages: "Split-KV: Breaking the Context Parallelism
 * Bottleneck in Diffusion Drafter Training", lede and "Split-KV's Core
 * Mechanism"; arXiv:2611.05926, Abstract):  the draft tokens, a few blocks
 * placed at sampled anchor positions, attend to a context many times their
 * length, each block to a part of it only.  The context K/V stays resident in
 * chunks; every chunk yields a query-sized partial result and the partials
 * are merged exactly, so the
 * result equals unsharded attention.  The backward reuses the merged
 * log-sum-exp.  Work items are placed on persistent workgroups by a
 * cost-aware longest-processing-time-first (LPT) planner ("LPT Scheduling").
 *
 * Mask reading (skv_problem.mask): draft block b of a sequence is anchored
 * at context position a_b.
 *  - SKV_MASK_PREFIX (default): its `block` query rows see the context
 *    prefix [0, e_b) with e_b = min(a_b + block, N_s) (the block's own tokens
 *    are context positions a_b .. a_b + block - 1).
 *  - SKV_MASK_OWN_BLOCK: its rows see the context prefix [0, e_b) with
 *    e_b = min(a_b, N_s), plus all `block` keys of the block's own draft
 *    tokens, a query-sized K/V segment passed separately (k_own, v_own:
 *    [sum_s Mq_s, hkv, d], row t = draft token t).  Its contribution is one
 *    more partial per sequence (sparse_attn_own_fwd), merged like the rest.
 * Anchors are sorted ascending per sequence.
 *
 * Conventions shared by every call:
 *  - All device pointers are caller-owned; the library never allocates,
 *    frees or synchronizes.  Device calls are asynchronous on `stream`
 *    (a hipStream_t; NULL = the default stream): the buffers a call reads
 *    (inputs and plan arrays) must hold their contents, and every buffer must
 *    stay allocated, until that work completes, and writes to them issued on
 *    other streams (a plan upload, say) must be ordered before it by the
 *    caller.  Host calls (planning, sizing) are synchronous, pure, and touch
 *    no GPU.
 *  - A pointer may be NULL only for a buffer with no rows: query-sized ones
 *    (Q, O, dO, dQ, LSE, partials, own-block tensors) when the batch has no
 *    query rows, context-sized ones (K, V, dK, dV) when it has no context.
 *  - Return value: SKV_OK or a negative skv_status; the reason is available
 *    from skv_last_error() on the calling thread.  Arguments are validated
 *    before any HIP call, so validation errors leave the stream untouched.
 *    A HIP launch failure returns SKV_EHIP.  Faults inside kernels surface
 *    at the caller's next synchronization.
 *  - Q, dO, O, dQ:   [sum_s Mq_s, hq, d]   element (t, h, x) at
 *                    t*q_stride_tok + h*q_stride_head + x
 *    K, V, dK, dV:   [sum_s N_s, hkv, d]   element (j, g, x) at
 *                    j*kv_stride_tok + g*kv_stride_head + x
 *    LSE:            float [sum_s Mq_s, hq], row-major (t*hq + h).
 *    Token and head strides are at least d (rows do not overlap) and
 *    multiples of 16 bytes.  For bf16, one sequence's K/V rows must span at
 *    most 2^31 bytes (N_s * kv_stride_tok * 2); larger sequences are
 *    rejected (SKV_ESHAPE).
 *  - Query head h uses KV head h / (hq / hkv).
 *  - Logits are sm_scale * q.k; LSE is in natural-log units.
 */
#ifndef SPLITKV_H_
#define SPLITKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_EINVAL = -1,     /* null pointer, bad count, unsorted anchors, ... */
  SKV_EDTYPE = -2,     /* dtype not supported by this call */
  SKV_ESHAPE = -3,     /* head_dim, head counts, chunk, strides or alignment */
  SKV_EHIP = -4,       /* a HIP runtime call failed */
  SKV_EWORKSPACE = -5, /* workspace missing or too small */
  SKV_EPLAN = -6       /* plan does not match the call */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;
typedef enum { SKV_ITEM_FWD = 0, SKV_ITEM_BWD = 1 } skv_item_kind;
typedef enum { SKV_POLICY_LPT = 0, SKV_POLICY_STATIC = 1 } skv_policy;

enum { SKV_TILE = 64 }; /* key-tile granularity of mask skipping and of the cost model */

/* One attention problem: a batch of n_seq sequences packed along the token
 * axis.  Sequence s owns query rows [q_off[s], q_off[s+1]) (a whole number of
 * draft blocks) and context tokens [kv_off[s], kv_off[s+1]).  Its draft block
 * b (0-based within s) is anchor[q_off[s]/block + b].  Every pointer pair holds
 * the same values in host memory (h_*) and device memory (d_*). */
typedef enum { SKV_MASK_PREFIX = 0, SKV_MASK_OWN_BLOCK = 1 } skv_mask;

typedef struct skv_problem {
  int32_t n_seq;
  int32_t block;          /* B: draft tokens per anchor, >= 1 */
  int32_t hq;             /* query heads */
  int32_t hkv;            /* KV heads; hq % hkv == 0 */
  int32_t d;              /* head dim: 128 for bf16; 64 or 128 for f32 */
  int32_t chunk;          /* L: KV chunk length, positive multiple of SKV_TILE */
  int32_t dtype;          /* skv_dtype of Q, K, V, O, dO, dQ, dK, dV */
  float sm_scale;         /* logit scale, finite and > 0 (usually 1/sqrt(d)) */
  int32_t mask;           /* skv_mask: SKV_MASK_PREFIX (0) or SKV_MASK_OWN_BLOCK */
  int32_t reserved;       /* 0 */
  const int64_t *h_q_off, *d_q_off;    /* [n_seq+1], multiples of block, non-decreasing, q_off[0] = 0 */
  const int64_t *h_kv_off, *d_kv_off;  /* [n_seq+1], non-decreasing */
  const int32_t *h_anchor, *d_anchor;  /* [q_off[n_seq]/block], 0 <= a <= 2^31-1-block, sorted per sequence;
                                        anchors past the context act as N (the whole context) */
  int64_t q_stride_tok, q_stride_head;   /* elements; head_dim is contiguous */
  int64_t kv_stride_tok, kv_stride_head; /* elements; head_dim is contiguous */
} skv_problem;

/* One work item, 40 bytes.  Built on the host by skv_item_table (and
 * skv_coarsen_fwd_items).
 * FWD: (seq, kv_head, chunk, range) covers draft blocks [lo, hi) of the
 *      sequence, all hq/hkv query heads of kv_head, against the n_chunk
 *      consecutive chunks chunk .. chunk + n_chunk - 1 (one contiguous key
 *      range); part_base is the first partial row of (seq, chunk), where the
 *      item writes the one partial of all its chunks.
 * BWD: covers context keys [lo, hi) of the sequence (inside chunk `chunk`)
 *      for kv_head; part_base is unused (0); n_chunk is 1.
 * skv_item_table sets n_chunk = 1; kernels treat n_chunk < 1 as 1. */
typedef struct skv_item {
  int32_t seq, kv_head, chunk, range;
  int64_t part_base;
  int32_t lo, hi;
  int32_t n_chunk, reserved;
} skv_item;

/* A plan as the kernels read it: items grouped by persistent workgroup.
 * Worker w's list is d_items[d_worker_off[w] .. d_worker_off[w+1]), in the
 * order the planner assigned them.  n_workers is the launched grid size.
 * Each worker claims the items of its own list in order through the atomic
 * cursor d_claim[w]; once its list is exhausted it claims the remaining
 * items of the other lists (the next workers first), so a slow compute unit
 * delays the call by at most the item it holds; a count of the items claimed
 * so far lets a worker stop as soon as every item is taken.  Every item is
 * processed exactly once.  d_claim is caller-owned scratch of n_workers + 1
 * int32 (the cursors, then the count) that the library resets at the start of
 * every call; two calls in flight at the same time must not share it.  The
 * lists hold d_worker_off[n_workers] items, fewer than 2^31.
 * flags: SKV_PLAN_NO_STEAL makes every worker run exactly its own list (the
 * plan's assignment as computed, for measuring a plan's balance); the fp32
 * forward never steals.  d_ticks (optional, NULL = off): device int64
 * [n_workers]; the call writes each worker's busy time, from its start to
 * finding no more work, in ticks of the 100 MHz s_memrealtime clock. */
enum { SKV_PLAN_NO_STEAL = 1 };
typedef struct skv_plan {
  int32_t kind;       /* skv_item_kind */
  int32_t n_workers;  /* >= 1 */
  int64_t n_items;
  const skv_item* d_items;      /* device, [n_items] */
  const int64_t* d_worker_off;  /* device, [n_workers+1], d_worker_off[0] = 0 */
  int32_t* d_claim;             /* device scratch, [n_workers + 1] */
  int32_t flags;                /* 0 or SKV_PLAN_NO_STEAL */
  int32_t reserved;             /* 0 */
  int64_t* d_ticks;             /* device, [n_workers], optional */
} skv_plan;

/* Thread-local description of the last error (never NULL). */
const char* skv_last_error(void);

/* Validate a problem (host copies only).  SKV_OK if usable by the device calls. */
int skv_check_problem(const skv_problem* p);

/* Partial layout of sparse_attn_partial_fwd.  Sequence s has
 * n_chunk[s] = C_s = ceil(N_s / chunk) context partials, plus one (index C_s,
 * written by sparse_attn_own_fwd) under SKV_MASK_OWN_BLOCK; partial (s, c)
 * owns rows part_base[s] + c*hq*Mq_s + h*Mq_s + r  (h = query head, r = query
 * row in s).  part_base has n_seq+1 entries; part_base[n_seq] is the total
 * number of partial rows.  Either output may be NULL. */
int skv_partial_layout(const skv_problem* p, int64_t* part_base, int32_t* n_chunk);

/* Work items of a problem, in enumeration order (seq, kv_head, chunk, range),
 * row-major.  FWD: granule = draft blocks per item.  BWD: granule = keys per
 * item, a positive multiple of SKV_TILE; ranges restart at every chunk.
 * Cost = (hq/hkv) x number of (draft block, 64-key tile) pairs of the item in
 * which the block sees at least one key of the tile (block b sees tile t iff
 * t*64 < e_b) — the item's realized attention cost.  tok_start = token offset
 * of the item in the stream of (seq, kv_head, chunk) units laid end to end
 * (all FWD ranges of one unit share its start); *total_tok = length of that
 * stream.  Call with items == cost == tok_start == NULL to get *n_items only.
 * Output arrays, when given, hold *n_items entries. */
int skv_item_table(const skv_problem* p, int32_t kind, int32_t granule, skv_item* items, int64_t* cost,
                   int64_t* tok_start, int64_t* n_items, int64_t* total_tok);

/* Cost-aware longest-processing-time-first planning ("LPT Scheduling": sort
 * by cost, largest first, give each to the least-loaded worker).  Tie-break:
 * items in order of (cost descending, item id ascending); the chosen worker is
 * the one with the smallest (load, worker id).  Zero costs are planned too.
 * cost[n] >= 0.  Outputs (any may be NULL): assign[n] worker of each item;
 * order[n] item ids grouped by worker, each worker's items in assignment
 * order; worker_off[n_workers+1]; load[n_workers].  Host only. */
int lpt_plan(const int64_t* cost, int64_t n, int32_t n_workers, int32_t* assign, int64_t* order,
             int64_t* worker_off, int64_t* load);

/* Static token-count plan (the baseline LPT is compared with): worker of item
 * i = floor(tok_start[i] * n_workers / total_tok).  order/worker_off group the
 * items by worker in ascending id order.  Outputs may be NULL.  Host only. */
int skv_static_plan(const int64_t* tok_start, int64_t n, int64_t total_tok, int32_t n_workers,
                    int32_t* assign, int64_t* order, int64_t* worker_off);

/* items_out[i] = items[order[i]] for i < n (host gather into plan order);
 * every order[i] must lie in [0, n_items). */
int skv_gather_items(const skv_item* items, int64_t n_items, const int64_t* order, int64_t n, skv_item* items_out);

/* Drop zero-cost items from a plan's worker lists (host, pure).  A forward
 * item of zero cost has no row that sees any key of its chunk: its only
 * output is m_part = lse_part = -inf for its rows, which
 * sparse_attn_partial_fwd writes for every partial row before it runs the
 * plan.  Left in the lists they all land on one worker under LPT (they do not
 * change any load), which then runs thousands of empty items.  Inputs are
 * lpt_plan / skv_static_plan outputs (order [n], worker_off [n_workers+1]);
 * writes order_out [n] (first *n_out used) and worker_off_out
 * [n_workers+1], keeping the order within each list.  Backward plans must
 * keep their zero-cost items (they write the zero dK, dV of unseen keys). */
int skv_drop_zero_cost(const int64_t* cost, int64_t n, int32_t n_workers, const int64_t* order,
                       const int64_t* worker_off, int64_t* order_out, int64_t* worker_off_out, int64_t* n_out);

/* Local merge of chunks before the exchange (host, pure).  The pages' ranks
 * each aggregate the attention results of the KV they hold before the
 * query-sized exchange (Split-KV article, "Split-KV's Core Mechanism"); here a
 * forward item may likewise cover several consecutive chunks of the same rows
 * and emit a single partial for them, so rows get fewer partials to write and
 * merge.  Input: single-chunk FWD items (n_chunk == 1) with their costs, e.g.
 * skv_item_table output or a subset of it.  Items with equal (seq, kv_head,
 * lo, hi) form a group; in ascending chunk order each group is cut into runs:
 * a zero-cost item is emitted alone, and an item joins the open run iff its
 * chunk follows the run's last chunk and the run's cost is still below
 * `target` (>= 1).  Each run becomes one item (the first item's fields,
 * n_chunk = run length) whose cost is the sum.  Runs are written in the
 * order of their first item in the input.  items_out and cost_out hold n
 * entries; *n_out receives the count.  target = 1 leaves the table as is. */
int skv_coarsen_fwd_items(const skv_item* items, const int64_t* cost, int64_t n, int64_t target,
                          skv_item* items_out, int64_t* cost_out, int64_t* n_out);

/* Forward plan over chunk runs (host, pure): picks how long the runs of
 * skv_coarsen_fwd_items are and plans them with lpt_plan.  Longer runs mean
 * fewer partials to write and merge but coarser items, so the search starts
 * at rpw = runs_per_worker runs per worker and doubles rpw until LPT balances
 * the runs well enough:
 *   target = max(1, ceil(total / (n_workers * rpw)))   (double precision;
 *            total = sum of cost)
 *   runs   = skv_coarsen_fwd_items(items, cost, target)
 *   plan   = lpt_plan(run costs, n_workers)
 * stopping at the first rpw with max(load)/mean(load) - 1 <= max_imbalance
 * (mean in double precision), with rpw >= max_runs_per_worker, or with a
 * zero total.  Inputs as for skv_coarsen_fwd_items; runs_per_worker > 0,
 * max_runs_per_worker >= runs_per_worker, max_imbalance >= 0.  Outputs:
 * items_out, cost_out [n] (first *n_out used: the runs), order [n] (first
 * *n_out used: run indices grouped by worker), worker_off [n_workers+1],
 * load [n_workers], *rpw_used (the rpw of the returned plan).  Zero-cost runs
 * stay in the plan (skv_drop_zero_cost removes them). */
int skv_plan_fwd_runs(const skv_item* items, const int64_t* cost, int64_t n, int32_t n_workers,
                      double runs_per_worker, double max_runs_per_worker, double max_imbalance,
                      skv_item* items_out, int64_t* cost_out, int64_t* n_out, int64_t* order, int64_t* worker_off,
                      int64_t* load, double* rpw_used);

/* Forward partials, one per (sequence, KV chunk): the shard-local step of
 * Split-KV (article "Split-KV: Breaking the Context Parallelism Bottleneck in
 * Diffusion Drafter Training", section "Split-KV's Core Mechanism": each KV
 * shard stays where it is and computes attention of the full query set
 * against its own keys, giving a query-sized result).  For every query row r of
 * sequence s, query head h and chunk c with visible keys
 * J = {j in [c*L, min((c+1)*L, N_s)) : j < e_b}:
 *   m_part   = max_{j in J} s_j                        (s_j = sm_scale*q.k_j)
 *   o_part   = sum_{j in J} exp(s_j - m_part) * v_j    (unnormalised, fp32)
 *   lse_part = m_part + ln sum_{j in J} exp(s_j - m_part)
 * at row part_base[s] + c*hq*Mq_s + h*Mq_s + r (see skv_partial_layout);
 * o_part rows are d floats.  Rows with J empty get m_part = lse_part = -inf
 * and their o_part row is not written.  Fully masked 64-key tiles are never
 * read.  `plan` must be a FWD plan over skv_item_table items of this problem
 * covering every (seq, kv_head, chunk, range) of nonzero cost exactly once
 * (zero-cost items may be left out, see skv_drop_zero_cost): the call first
 * sets m_part and lse_part of every partial row to -inf, then runs the plan
 * with plan->n_workers workgroups.  Results are bitwise deterministic.
 * With items of several chunks (skv_coarsen_fwd_items) the partial of such an
 * item covers the keys of all its chunks and sits in its first chunk's rows;
 * the other chunks' rows stay -inf, and lse_merge gives the same result. */
int sparse_attn_partial_fwd(const skv_problem* p, const skv_plan* plan, const void* q, const void* k,
                            const void* v, float* o_part, float* m_part, float* lse_part, void* stream);

/* The own-block partial of every draft row (SKV_MASK_OWN_BLOCK only): for
 * row r of block b, query head h and the block's own keys J (its `block`
 * draft tokens, KV head h / (hq/hkv)), the same m_part / o_part / lse_part
 * formulas as above, written at partial index C_s of the sequence
 * (skv_partial_layout).  k_own, v_own: [sum Mq, hkv, d] in the problem dtype,
 * element (t, g, x) at t*own_stride_tok + g*own_stride_head + x (strides
 * 16-byte multiples).  Call after sparse_attn_partial_fwd on the same stream
 * (that call first sets every partial row to -inf).  Own-block limits:
 * block <= 64 and (hq/hkv) * block * block <= 8192 (SKV_ESHAPE otherwise).
 * Bitwise deterministic. */
int sparse_attn_own_fwd(const skv_problem* p, const void* q, const void* k_own, const void* v_own,
                        int64_t own_stride_tok, int64_t own_stride_head, float* o_part, float* m_part,
                        float* lse_part, void* stream);

/* Exact log-sum-exp merge of n_part partials of one sequence: the exact
 * aggregation of the shard results (article "Split-KV: Breaking the Context
 * Parallelism Bottleneck in Diffusion Drafter Training", section "Split-KV's
 * Core Mechanism": the query-sized results are combined exactly, so the
 * output equals attention over the unsharded context).
 * Inputs: o_part [n_part][hq][mq][d], m_part and lse_part [n_part][hq][mq]
 * (fp32, the layout sparse_attn_partial_fwd writes for one sequence: pass
 * pointers offset to part_base[s]).  Per row (h, r):
 *   M = max_c lse_c,  LSE = M + ln sum_c exp(lse_c - M),
 *   O = sum_{c : lse_c > -inf} exp(m_c - LSE) * o_c
 * (o_c rows of partials with lse_c = -inf are never read).  A row with every
 * lse_c = -inf gets O = 0 and LSE = -inf.  O is written in out_dtype at
 * o_out + r*o_stride_tok + h*o_stride_head (+ x); LSE at lse_out[r*lse_stride_tok + h].
 * n_part may be 0.  Bitwise deterministic. */
int lse_merge(int32_t n_part, int32_t hq, int64_t mq, int32_t d, const float* o_part, const float* m_part,
              const float* lse_part, void* o_out, int64_t o_stride_tok, int64_t o_stride_head, int32_t out_dtype,
              float* lse_out, int64_t lse_stride_tok, void* stream);

/* lse_merge of every sequence of a problem in one launch: the partials in
 * the layout of skv_partial_layout (d_part_base: its part_base array
 * [n_seq+1], copied to the device by the caller), O written in the problem
 * dtype with the Q layout, LSE as float [sum Mq][hq].  Per row the same
 * arithmetic, in the same order, as lse_merge on that row's sequence, so the
 * results are bitwise equal. */
int lse_merge_all(const skv_problem* p, const int64_t* d_part_base, const float* o_part, const float* m_part,
                  const float* lse_part, void* o_out, float* lse_out, void* stream);

/* Bytes of device workspace sparse_attn_bwd needs (256-byte aligned pieces):
 * fp32 dQ partials in the layout of skv_partial_layout ([rows][d]) and an
 * int32 run length per partial row; bf16
 * copies of Q and dO and fp32 LSE, Delta and int32 prefix ends in the
 * backward's packed row order; n_seq+1 int64 partial offsets.  0 for an
 * invalid problem. */
size_t skv_bwd_workspace_bytes(const skv_problem* p);

/* Backward of O with respect to Q, K, V, reusing the merged LSE (article
 * "Split-KV: Breaking the Context Parallelism Bottleneck in Diffusion Drafter
 * Training", section "Split-KV's Core Mechanism": the sharded result equals
 * the unsharded one, which the article ties to correct gradients in training;
 * so the backward works from the merged statistics as unsharded attention
 * would).
 * With P = exp(s - LSE) on visible entries (0 elsewhere), Delta = sum_x dO*O,
 * dS = P*(dO.v - Delta):  dV_j = sum P dO,  dQ = sm_scale * dS K,
 * dK_j = sm_scale * sum dS q, summed over the query heads of each KV head.
 * o = merged output (problem dtype, Q layout), lse = merged LSE (float
 * [sum Mq][hq]), dout = dO.  Outputs dq (Q layout), dk and dv (K/V layout)
 * are fully written, dk = dv = 0 for keys no query sees.  Every tensor
 * pointer (q, k, v, o, dout, dq, dk, dv) must be 16-byte aligned
 * (SKV_ESHAPE otherwise).
 * plan_kv is a BWD plan (key ranges; dK, dV are owned by their item);
 * plan_q is a FWD plan over the forward's items or chunk runs
 * (skv_coarsen_fwd_items): each item writes one dQ partial for all its
 * chunks, in its first chunk's rows, and the partials a row sees are summed
 * afterwards (plan_q must cover every nonzero-cost item exactly once).  The two plans need distinct claim
 * arrays.  No atomics: the result is bitwise reproducible.
 * Only SKV_BF16 with d = 128 is supported.
 * Under SKV_MASK_OWN_BLOCK `own` is required: its keys and values enter P and
 * dS like the context keys each row sees, their gradients
 * dk_own = sm_scale * sum dS q and dv_own = sum P dO (summed over the block's
 * rows and the query heads of each KV head) are written to own->dk, own->dv
 * (k_own layout, fully written), and their share of dQ joins the sum.  NULL
 * otherwise. */
typedef struct skv_own_block {
  const void* k;              /* [sum Mq, hkv, d] own-block keys (problem dtype) */
  const void* v;              /* own-block values, same layout */
  void* dk;                   /* outputs, same layout */
  void* dv;
  int64_t stride_tok, stride_head;  /* elements, 16-byte multiples, stride_head >= d */
} skv_own_block;

int sparse_attn_bwd(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                    const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                    void* dk, void* dv, void* workspace, size_t workspace_bytes, const skv_own_block* own,
                    void* stream);

/* sparse_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks and results as sparse_attn_bwd, without the
 * workspace: the library keeps it in a static device array of
 * SKV_NOALLOC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds
 * from its first such call until the process ends.  The call allocates and
 * frees nothing; problems whose skv_bwd_workspace_bytes exceeds the array are
 * rejected with SKV_EWORKSPACE before any device work.  The stream must belong
 * to the device current on the calling thread.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, or
 * other threads) race and must be serialized by the caller; calls in order on
 * one stream are safe.  Nothing in the array needs to start at zero: each call
 * writes every part it later reads. */
enum { SKV_NOALLOC_SCRATCH_BYTES = 64 << 20 };
int sparse_attn_bwd_noalloc(const skv_problem* p, const skv_plan* plan_kv, const skv_plan* plan_q, const void* q,
                            const void* k, const void* v, const void* o, const float* lse, const void* dout,
                            void* dq, void* dk, void* dv, const skv_own_block* own, void* stream);

/* ---- Instrumentation (host) ----
 * Per-kernel timing with HIP events, off by default.  While enabled, every
 * kernel the library launches is bracketed by two events recorded on the
 * stream it is launched on (the library creates and reuses the events; this
 * adds a few microseconds per launch and must stay off under graph capture).
 * skv_timing_collect waits for every recorded event, writes per kernel name
 * the number of launches and their summed event-to-event time into
 * out[0 .. min(max_entries, *n_entries)) and resets the tallies; *n_entries
 * receives the number of kernels with at least one launch.  Kernel names:
 * "fill_partials" (also resets the forward plan's claim cursors), "partial_fwd_bf16",
 * "partial_fwd_f32", "lse_merge", "bwd_pack" (also resets the backward plans'
 * claim cursors and finds the partial offsets), "bwd_kv", "bwd_dq",
 * "bwd_finalize", "own_fwd", "own_bwd". */
typedef struct skv_kernel_time {
  const char* name;   /* static string */
  int64_t launches;
  double total_ms;
} skv_kernel_time;
int skv_timing_enable(int32_t on);
int skv_timing_collect(skv_kernel_time* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_H_ */
