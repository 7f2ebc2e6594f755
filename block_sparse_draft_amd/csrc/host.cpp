// Host side of libsplitkv: argument validation, the error channel, the
// partial layout, the realized-cost work-item table, and the LPT and static
// planners.  Nothing here touches a GPU.
//
// Planning follows the LPT description on the Split-KV article page
// ("LPT Scheduling": sort by processing time, longest first, each task to the
// least-loaded machine) with the processing time replaced by the realized
// attention cost of each item, which the global query view makes observable
// ("Split-KV's Core Mechanism"; arXiv:2611.05926, Abstract).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "internal.h"

namespace skv {

static thread_local std::string g_last_error = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error = "no error"; }

const char* last_error_cstr() { return g_last_error.c_str(); }

}  // namespace skv

using namespace skv;

extern "C" const char* skv_last_error(void) { return last_error_cstr(); }

extern "C" int skv_check_problem(const skv_problem* p) {
  if (!p) return fail(SKV_EINVAL, "problem is NULL");
  if (p->n_seq < 0) return fail(SKV_EINVAL, "n_seq = %d < 0", p->n_seq);
  if (p->block < 1) return fail(SKV_EINVAL, "block = %d < 1", p->block);
  if (p->hq < 1 || p->hkv < 1) return fail(SKV_ESHAPE, "hq = %d, hkv = %d must be >= 1", p->hq, p->hkv);
  if (p->hq % p->hkv) return fail(SKV_ESHAPE, "hq = %d is not a multiple of hkv = %d", p->hq, p->hkv);
  if ((int64_t)p->block * (p->hq / p->hkv) > (1 << 20)) return fail(SKV_ESHAPE, "block * hq/hkv exceeds 2^20");
  if (p->dtype != SKV_F32 && p->dtype != SKV_BF16) return fail(SKV_EDTYPE, "unknown dtype %d", p->dtype);
  if (p->mask != SKV_MASK_PREFIX && p->mask != SKV_MASK_OWN_BLOCK) return fail(SKV_EINVAL, "unknown mask %d", p->mask);
  if (p->dtype == SKV_BF16 && p->d != 128) return fail(SKV_ESHAPE, "bf16 supports head_dim 128, got %d", p->d);
  if (p->dtype == SKV_F32 && p->d != 64 && p->d != 128)
    return fail(SKV_ESHAPE, "f32 supports head_dim 64 or 128, got %d", p->d);
  if (p->chunk < SKV_TILE || p->chunk % SKV_TILE)
    return fail(SKV_ESHAPE, "chunk = %d must be a positive multiple of %d", p->chunk, SKV_TILE);
  if (!(std::isfinite(p->sm_scale) && p->sm_scale > 0.f))
    return fail(SKV_EINVAL, "sm_scale must be finite and > 0");
  if (!p->h_q_off || !p->h_kv_off) return fail(SKV_EINVAL, "host offset arrays are NULL");
  if (!p->h_anchor && p->h_q_off[p->n_seq] > 0) return fail(SKV_EINVAL, "host anchor array is NULL");
  // Vector loads move 16 bytes: strides must keep every head row 16-byte aligned.
  const int64_t vec = p->dtype == SKV_BF16 ? 8 : 4;
  // Token and head strides of at least d keep every (token, head) row of d
  // elements apart from the others, which the kernels' buffer ranges (one
  // sequence's rows from its first key) rely on.
  if (p->q_stride_head < p->d || p->kv_stride_head < p->d || p->q_stride_tok < p->d || p->kv_stride_tok < p->d)
    return fail(SKV_ESHAPE, "token and head strides must be >= d");
  if (p->q_stride_tok % vec || p->q_stride_head % vec || p->kv_stride_tok % vec || p->kv_stride_head % vec)
    return fail(SKV_ESHAPE, "strides must be multiples of %lld elements (16 bytes)", (long long)vec);
  // Query rows start at row 0: the kernels that walk every row of the batch
  // (packing, merge, finalize, own-block) index rows from 0 up to q_off[n_seq].
  if (p->h_q_off[0] != 0) return fail(SKV_EINVAL, "q_off[0] = %lld must be 0", (long long)p->h_q_off[0]);
  if (p->h_kv_off[0] < 0) return fail(SKV_EINVAL, "kv_off[0] must be >= 0");
  for (int s = 0; s < p->n_seq; ++s) {
    const int64_t q0 = p->h_q_off[s], q1 = p->h_q_off[s + 1];
    const int64_t k0 = p->h_kv_off[s], k1 = p->h_kv_off[s + 1];
    if (q1 < q0 || k1 < k0) return fail(SKV_EINVAL, "offsets of sequence %d decrease", s);
    if (q0 % p->block || q1 % p->block)
      return fail(SKV_EINVAL, "query offsets of sequence %d are not multiples of block %d", s, p->block);
    if (k1 - k0 > (int64_t)INT32_MAX - p->block) return fail(SKV_ESHAPE, "sequence %d is too long", s);
    // bf16 kernels address one sequence's K/V rows with 32-bit byte offsets
    if (p->dtype == SKV_BF16 && (k1 - k0) * p->kv_stride_tok * 2 > (int64_t)INT32_MAX)
      return fail(SKV_ESHAPE, "sequence %d spans more than 2^31 bytes of K/V rows", s);
    const SeqView v = seq_view(p, s);
    for (int64_t b = 0; b < v.n_blk; ++b) {
      const int32_t a = p->h_anchor[v.blk0 + b];
      if (a < 0) return fail(SKV_EINVAL, "anchor %lld of sequence %d is negative", (long long)b, s);
      // kernels form a + block in 32-bit arithmetic
      if (a > INT32_MAX - p->block)
        return fail(SKV_EINVAL, "anchor %lld of sequence %d exceeds 2^31 - 1 - block", (long long)b, s);
      if (b > 0 && a < p->h_anchor[v.blk0 + b - 1])
        return fail(SKV_EINVAL, "anchors of sequence %d are not sorted ascending", s);
    }
  }
  return SKV_OK;
}

extern "C" int skv_partial_layout(const skv_problem* p, int64_t* part_base, int32_t* n_chunk) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  int64_t base = 0;
  for (int s = 0; s < p->n_seq; ++s) {
    const SeqView v = seq_view(p, s);
    const int64_t c = n_partials(p, v.n);
    if (part_base) part_base[s] = base;
    if (n_chunk) n_chunk[s] = (int32_t)c;
    base += c * p->hq * v.mq;
  }
  if (part_base) part_base[p->n_seq] = base;
  return SKV_OK;
}

// Number of 64-key tiles t in [t0, t1) with t*64 < e: the tiles of that span in
// which a block with prefix end e sees at least one key.
static inline int64_t tiles_seen(int64_t e, int64_t t0, int64_t t1) {
  const int64_t last = ceil_div(e, SKV_TILE);  // tiles 0 .. last-1 start below e
  return std::max<int64_t>(0, std::min(last, t1) - t0);
}

extern "C" int skv_item_table(const skv_problem* p, int32_t kind, int32_t granule, skv_item* items, int64_t* cost,
                              int64_t* tok_start, int64_t* n_items, int64_t* total_tok) {
  int rc = skv_check_problem(p);
  if (rc) return rc;
  if (kind != SKV_ITEM_FWD && kind != SKV_ITEM_BWD) return fail(SKV_EINVAL, "unknown item kind %d", kind);
  if (granule < 1) return fail(SKV_EINVAL, "granule = %d < 1", granule);
  if (kind == SKV_ITEM_BWD && granule % SKV_TILE)
    return fail(SKV_EINVAL, "bwd granule = %d is not a multiple of %d", granule, SKV_TILE);
  const int64_t G = p->hq / p->hkv;
  int64_t n = 0, tok = 0, base = 0;
  std::vector<int64_t> ends, seq_cost;
  for (int s = 0; s < p->n_seq; ++s) {
    const SeqView v = seq_view(p, s);
    const int64_t C = ceil_div(v.n, p->chunk);
    ends.resize(v.n_blk);
    for (int64_t b = 0; b < v.n_blk; ++b)
      ends[b] = std::min<int64_t>((int64_t)p->h_anchor[v.blk0 + b] + end_shift(p), v.n);
    // Items per chunk, and the cost of each (chunk, range): the same for every
    // KV head, so it is computed once per sequence.
    const int64_t nr_fwd = ceil_div(v.n_blk, granule);
    const int64_t nr_max = kind == SKV_ITEM_FWD ? nr_fwd : ceil_div(std::min<int64_t>(p->chunk, v.n), granule);
    if (cost) {
      seq_cost.assign(C * nr_max, 0);
      for (int64_t c = 0; c < C; ++c) {
        const int64_t lo = c * p->chunk, hi = std::min<int64_t>(lo + p->chunk, v.n);
        if (kind == SKV_ITEM_FWD) {
          const int64_t t0 = lo / SKV_TILE, t1 = ceil_div(hi, SKV_TILE);
          for (int64_t r = 0; r < nr_fwd; ++r) {
            const int64_t b0 = r * granule, b1 = std::min<int64_t>(b0 + granule, v.n_blk);
            int64_t sum = 0;
            for (int64_t b = b0; b < b1; ++b) sum += tiles_seen(ends[b], t0, t1);
            seq_cost[c * nr_max + r] = G * sum;
          }
        } else {
          const int64_t nr = ceil_div(hi - lo, granule);
          for (int64_t r = 0; r < nr; ++r) {
            const int64_t klo = lo + r * granule, khi = std::min<int64_t>(klo + granule, hi);
            const int64_t t0 = klo / SKV_TILE, t1 = ceil_div(khi, SKV_TILE);
            int64_t sum = 0;
            for (int64_t b = 0; b < v.n_blk; ++b) sum += tiles_seen(ends[b], t0, t1);
            seq_cost[c * nr_max + r] = G * sum;
          }
        }
      }
    }
    for (int g = 0; g < p->hkv; ++g) {
      for (int64_t c = 0; c < C; ++c) {
        const int64_t lo = c * p->chunk, hi = std::min<int64_t>(lo + p->chunk, v.n);
        const int64_t nr = kind == SKV_ITEM_FWD ? nr_fwd : ceil_div(hi - lo, granule);
        for (int64_t r = 0; r < nr; ++r) {
          if (cost) cost[n] = seq_cost[c * nr_max + r];
          if (kind == SKV_ITEM_FWD) {
            const int64_t b0 = r * granule, b1 = std::min<int64_t>(b0 + granule, v.n_blk);
            if (tok_start) tok_start[n] = tok;
            if (items)
              items[n] = skv_item{s, g, (int32_t)c, (int32_t)r, base + c * p->hq * v.mq, (int32_t)b0, (int32_t)b1, 1, 0};
          } else {
            const int64_t klo = lo + r * granule, khi = std::min<int64_t>(klo + granule, hi);
            if (tok_start) tok_start[n] = tok + (klo - lo);
            if (items) items[n] = skv_item{s, g, (int32_t)c, (int32_t)r, 0, (int32_t)klo, (int32_t)khi, 1, 0};
          }
          ++n;
        }
        tok += hi - lo;
      }
    }
    base += n_partials(p, v.n) * p->hq * v.mq;  // chunks, then the own-block partial if any
  }
  if (n_items) *n_items = n;
  if (total_tok) *total_tok = tok;
  return SKV_OK;
}

static int write_csr(const std::vector<std::vector<int64_t>>& lists, int64_t* order, int64_t* worker_off) {
  int64_t pos = 0;
  if (worker_off) worker_off[0] = 0;
  for (size_t w = 0; w < lists.size(); ++w) {
    for (int64_t i : lists[w]) {
      if (order) order[pos] = i;
      ++pos;
    }
    if (worker_off) worker_off[w + 1] = pos;
  }
  return SKV_OK;
}

// Stable sort of idx by key(i) ascending (key values in [0, max_key]): LSD
// radix, 8 bits per pass, so equal keys keep their order in idx.
template <class Key>
static void radix_sort_by(std::vector<int64_t>& idx, uint64_t max_key, Key key) {
  std::vector<int64_t> tmp(idx.size());
  for (int shift = 0; shift < 64 && (max_key >> shift) != 0; shift += 8) {
    int64_t cnt[257] = {0};
    for (int64_t i : idx) ++cnt[((key(i) >> shift) & 255) + 1];
    for (int d = 0; d < 256; ++d) cnt[d + 1] += cnt[d];
    for (int64_t i : idx) tmp[cnt[(key(i) >> shift) & 255]++] = i;
    idx.swap(tmp);
  }
}

static int bit_width(uint64_t x) {
  int b = 0;
  while (b < 64 && (x >> b) != 0) ++b;
  return b;
}

extern "C" int lpt_plan(const int64_t* cost, int64_t n, int32_t n_workers, int32_t* assign, int64_t* order,
                        int64_t* worker_off, int64_t* load) {
  if (n < 0) return fail(SKV_EINVAL, "n = %lld < 0", (long long)n);
  if (n_workers < 1) return fail(SKV_EINVAL, "n_workers = %d < 1", n_workers);
  if (n > 0 && !cost) return fail(SKV_EINVAL, "cost is NULL");
  for (int64_t i = 0; i < n; ++i)
    if (cost[i] < 0) return fail(SKV_EINVAL, "cost[%lld] < 0", (long long)i);
  // Longest first; equal costs keep ascending item id.
  int64_t max_cost = 0, total = 0;
  for (int64_t i = 0; i < n; ++i) {
    max_cost = std::max(max_cost, cost[i]);
    total = cost[i] > INT64_MAX - total ? INT64_MAX : total + cost[i];
  }
  std::vector<int64_t> seq(n);
  for (int64_t i = 0; i < n; ++i) seq[i] = i;
  radix_sort_by(seq, (uint64_t)max_cost, [&](int64_t i) { return (uint64_t)(max_cost - cost[i]); });
  // Min-heap of (load, worker): the top is the least-loaded worker, lowest id
  // on ties.  Each item replaces the top and sifts it down.  When every load
  // fits, a worker's slot is one integer, load * 2^wb + worker.
  std::vector<int32_t> owner(n);
  std::vector<int64_t> count(n_workers + 1, 0);
  std::vector<int64_t> final_load(n_workers, 0);
  const int wb = bit_width((uint64_t)(n_workers - 1));
  const size_t H = (size_t)n_workers;
  if (wb < 62 && total < (INT64_C(1) << (62 - wb))) {
    // A 4-ary heap (children of k: 4k+1 .. 4k+4): half the levels of a
    // binary one.  Slots are distinct, so the top is the same either way.
    // Missing children read as UINT64_MAX (the array is padded to a
    // multiple of 4 plus one).
    std::vector<uint64_t> heap(((H + 2) / 4) * 4 + 1 + 4, UINT64_MAX);
    for (size_t w = 0; w < H; ++w) heap[w] = (uint64_t)w;  // ascending: already a heap
    const uint64_t wmask = (UINT64_C(1) << wb) - 1;
    for (int64_t i : seq) {
      uint64_t top = heap[0];
      owner[i] = (int32_t)(top & wmask);
      top += (uint64_t)cost[i] << wb;
      size_t k = 0;
      for (;;) {
        const size_t c = 4 * k + 1;
        if (c >= H) break;
        size_t m = c;
        uint64_t mv = heap[c];
        if (heap[c + 1] < mv) { mv = heap[c + 1]; m = c + 1; }
        if (heap[c + 2] < mv) { mv = heap[c + 2]; m = c + 2; }
        if (heap[c + 3] < mv) { mv = heap[c + 3]; m = c + 3; }
        if (mv >= top) break;
        heap[k] = mv;
        k = m;
      }
      heap[k] = top;
    }
    heap.resize(H);
    for (uint64_t sl : heap) final_load[sl & wmask] = (int64_t)(sl >> wb);
  } else {
    struct Slot {
      int64_t load;
      int32_t w;
      bool operator<(const Slot& o) const { return load < o.load || (load == o.load && w < o.w); }
    };
    std::vector<Slot> heap(H);
    for (size_t w = 0; w < H; ++w) heap[w] = Slot{0, (int32_t)w};
    for (int64_t i : seq) {
      Slot top = heap[0];
      owner[i] = top.w;
      top.load += cost[i];
      size_t k = 0;
      for (;;) {
        size_t c = 2 * k + 1;
        if (c >= H) break;
        if (c + 1 < H && heap[c + 1] < heap[c]) ++c;
        if (!(heap[c] < top)) break;
        heap[k] = heap[c];
        k = c;
      }
      heap[k] = top;
    }
    for (const Slot& sl : heap) final_load[sl.w] = sl.load;
  }
  // CSR by worker; each list keeps the order the items were assigned in.
  for (int64_t i : seq) ++count[owner[i] + 1];
  for (int32_t w = 0; w < n_workers; ++w) count[w + 1] += count[w];
  if (worker_off) std::copy(count.begin(), count.end(), worker_off);
  if (load) std::copy(final_load.begin(), final_load.end(), load);
  std::vector<int64_t> pos(count.begin(), count.end() - 1);
  for (int64_t i : seq) {
    const int32_t w = owner[i];
    if (assign) assign[i] = w;
    if (order) order[pos[w]] = i;
    ++pos[w];
  }
  return SKV_OK;
}

extern "C" int skv_static_plan(const int64_t* tok_start, int64_t n, int64_t total_tok, int32_t n_workers,
                               int32_t* assign, int64_t* order, int64_t* worker_off) {
  if (n < 0) return fail(SKV_EINVAL, "n = %lld < 0", (long long)n);
  if (n_workers < 1) return fail(SKV_EINVAL, "n_workers = %d < 1", n_workers);
  if (n > 0 && !tok_start) return fail(SKV_EINVAL, "tok_start is NULL");
  std::vector<std::vector<int64_t>> lists(n_workers);
  for (int64_t i = 0; i < n; ++i) {
    if (tok_start[i] < 0 || (total_tok > 0 && tok_start[i] >= total_tok))
      return fail(SKV_EINVAL, "tok_start[%lld] outside [0, total_tok)", (long long)i);
    // 128-bit product: tok_start * n_workers may exceed 2^63 for huge streams.
    const int32_t w = total_tok > 0 ? (int32_t)((__int128)tok_start[i] * n_workers / total_tok) : 0;
    if (assign) assign[i] = w;
    lists[w].push_back(i);
  }
  return write_csr(lists, order, worker_off);
}

extern "C" int skv_gather_items(const skv_item* items, int64_t n_items, const int64_t* order, int64_t n,
                                skv_item* items_out) {
  if (n < 0 || n_items < 0) return fail(SKV_EINVAL, "negative count");
  if (n > 0 && (!items || !order || !items_out)) return fail(SKV_EINVAL, "NULL argument");
  for (int64_t i = 0; i < n; ++i) {
    if (order[i] < 0 || order[i] >= n_items) return fail(SKV_EINVAL, "order[%lld] out of range", (long long)i);
    items_out[i] = items[order[i]];
  }
  clear_error();
  return SKV_OK;
}

extern "C" int skv_drop_zero_cost(const int64_t* cost, int64_t n, int32_t n_workers, const int64_t* order,
                                  const int64_t* worker_off, int64_t* order_out, int64_t* worker_off_out,
                                  int64_t* n_out) {
  if (n < 0 || n_workers < 1) return fail(SKV_EINVAL, "bad counts n=%lld n_workers=%d", (long long)n, n_workers);
  if (!worker_off || !worker_off_out || !n_out || (n > 0 && (!cost || !order || !order_out)))
    return fail(SKV_EINVAL, "NULL argument");
  if (worker_off[0] != 0 || worker_off[n_workers] != n) return fail(SKV_EINVAL, "worker_off does not span n items");
  int64_t k = 0;
  worker_off_out[0] = 0;
  for (int32_t w = 0; w < n_workers; ++w) {
    if (worker_off[w + 1] < worker_off[w]) return fail(SKV_EINVAL, "worker_off decreases at %d", w);
    for (int64_t i = worker_off[w]; i < worker_off[w + 1]; ++i) {
      const int64_t it = order[i];
      if (it < 0 || it >= n) return fail(SKV_EINVAL, "order[%lld] out of range", (long long)i);
      if (cost[it] != 0) order_out[k++] = it;
    }
    worker_off_out[w + 1] = k;
  }
  *n_out = k;
  clear_error();
  return SKV_OK;
}

// Runs of consecutive chunks of the same rows become one forward item.
// Checks of a coarsening input: single-chunk items, costs >= 0, no negative field.
static int check_coarsen_input(const skv_item* items, const int64_t* cost, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const skv_item& t = items[i];
    if (t.n_chunk != 1 || cost[i] < 0)
      return fail(SKV_EINVAL, "item %lld: n_chunk %d, cost %lld (single-chunk items with cost >= 0 expected)",
                  (long long)i, t.n_chunk, (long long)cost[i]);
    if (t.seq < 0 || t.kv_head < 0 || t.lo < 0 || t.hi < 0 || t.chunk < 0)
      return fail(SKV_EINVAL, "item %lld has a negative field", (long long)i);
  }
  return SKV_OK;
}

// Item indices in group order (seq, kv_head, lo, hi, chunk), ties by index:
// one stable LSD radix sort, 8 bits per pass, over a composite key whose
// fields take the bit widths of their maxima (field by field when the widths
// add up to more than 64 bits).
static void group_order(const skv_item* items, int64_t n, std::vector<int64_t>& idx) {
  idx.resize(n);
  for (int64_t i = 0; i < n; ++i) idx[i] = i;
  int32_t skv_item::*const fields[5] = {&skv_item::seq, &skv_item::kv_head, &skv_item::lo, &skv_item::hi,
                                        &skv_item::chunk};
  int width[5], total = 0;
  for (int f = 0; f < 5; ++f) {
    uint32_t mx = 0;
    for (int64_t i = 0; i < n; ++i) mx = std::max(mx, (uint32_t)(items[i].*fields[f]));
    width[f] = bit_width(mx);
    total += width[f];
  }
  if (total > 64) {
    std::vector<uint32_t> field(n);
    for (int f = 4; f >= 0; --f) {  // last field first
      uint64_t mx = 0;
      for (int64_t i = 0; i < n; ++i) {
        field[i] = (uint32_t)(items[i].*fields[f]);
        mx = std::max<uint64_t>(mx, field[i]);
      }
      radix_sort_by(idx, mx, [&](int64_t i) { return (uint64_t)field[i]; });
    }
    return;
  }
  std::vector<uint64_t> key(n), key2(n);
  for (int64_t i = 0; i < n; ++i) {
    uint64_t kk = 0;
    for (int f = 0; f < 5; ++f) kk = (kk << width[f]) | (uint64_t)(uint32_t)(items[i].*fields[f]);
    key[i] = kk;
  }
  std::vector<int64_t> idx2(n);
  for (int shift = 0; shift < total; shift += 8) {
    int64_t cnt[257] = {0};
    for (int64_t i = 0; i < n; ++i) ++cnt[((key[i] >> shift) & 255) + 1];
    for (int d = 0; d < 256; ++d) cnt[d + 1] += cnt[d];
    for (int64_t i = 0; i < n; ++i) {
      const int64_t pos = cnt[(key[i] >> shift) & 255]++;
      key2[pos] = key[i];
      idx2[pos] = idx[i];
    }
    key.swap(key2);
    idx.swap(idx2);
  }
}

// Runs over items in group order `idx`: consecutive chunks of the same rows
// join a run while its cost is below `target`; a zero-cost item stands alone.
// Output in order of each run's first item.
static void build_runs(const skv_item* items, const int64_t* cost, int64_t n, const std::vector<int64_t>& idx,
                       int64_t target, skv_item* items_out, int64_t* cost_out, int64_t* n_out) {
  struct Run { int64_t first; int32_t len; int64_t cost; };
  std::vector<Run> runs;
  runs.reserve(n);
  bool open = false;
  for (int64_t j = 0; j < n; ++j) {
    const int64_t i = idx[j];
    const skv_item& t = items[i];
    bool join = false;
    if (open && cost[i] > 0) {
      const skv_item& f = items[runs.back().first];
      join = f.seq == t.seq && f.kv_head == t.kv_head && f.lo == t.lo && f.hi == t.hi &&
             t.chunk == f.chunk + runs.back().len && runs.back().cost < target;
    }
    if (join) {
      runs.back().len += 1;
      runs.back().cost += cost[i];
    } else {
      runs.push_back(Run{i, 1, cost[i]});
    }
    open = cost[i] > 0;  // a zero-cost item stands alone
  }
  // output in order of each run's first item (first items are distinct)
  std::vector<int64_t> run_of(n, -1);
  for (size_t r = 0; r < runs.size(); ++r) run_of[runs[r].first] = (int64_t)r;
  int64_t k = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (run_of[i] < 0) continue;
    const Run& R = runs[run_of[i]];
    items_out[k] = items[i];
    items_out[k].n_chunk = R.len;
    cost_out[k] = R.cost;
    ++k;
  }
  *n_out = k;
}

extern "C" int skv_coarsen_fwd_items(const skv_item* items, const int64_t* cost, int64_t n, int64_t target,
                                     skv_item* items_out, int64_t* cost_out, int64_t* n_out) {
  if (n < 0 || target < 1) return fail(SKV_EINVAL, "n = %lld, target = %lld", (long long)n, (long long)target);
  if (n > 0 && (!items || !cost || !items_out || !cost_out)) return fail(SKV_EINVAL, "NULL array");
  if (!n_out) return fail(SKV_EINVAL, "n_out is NULL");
  int rc = check_coarsen_input(items, cost, n);
  if (rc) return rc;
  std::vector<int64_t> idx;
  group_order(items, n, idx);
  build_runs(items, cost, n, idx, target, items_out, cost_out, n_out);
  return SKV_OK;
}

extern "C" int skv_plan_fwd_runs(const skv_item* items, const int64_t* cost, int64_t n, int32_t n_workers,
                                 double runs_per_worker, double max_runs_per_worker, double max_imbalance,
                                 skv_item* items_out, int64_t* cost_out, int64_t* n_out, int64_t* order,
                                 int64_t* worker_off, int64_t* load, double* rpw_used) {
  if (n < 0 || n_workers < 1) return fail(SKV_EINVAL, "bad counts n=%lld n_workers=%d", (long long)n, n_workers);
  if (!(runs_per_worker > 0.0) || !(max_runs_per_worker >= runs_per_worker) || !std::isfinite(max_runs_per_worker))
    return fail(SKV_EINVAL, "runs per worker %g, max %g", runs_per_worker, max_runs_per_worker);
  if (!(max_imbalance >= 0.0)) return fail(SKV_EINVAL, "max_imbalance must be >= 0");
  if (!n_out || !worker_off || !load || !rpw_used || (n > 0 && (!items || !cost || !items_out || !cost_out || !order)))
    return fail(SKV_EINVAL, "NULL argument");
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (cost[i] < 0) return fail(SKV_EINVAL, "cost[%lld] < 0", (long long)i);
    if (cost[i] > INT64_MAX - total) return fail(SKV_EINVAL, "total cost overflows");
    total += cost[i];
  }
  int rc = check_coarsen_input(items, cost, n);
  if (rc) return rc;
  std::vector<int64_t> idx;  // group order: the same for every target
  group_order(items, n, idx);
  double rpw = runs_per_worker;
  for (;;) {
    const double t = std::ceil((double)total / ((double)n_workers * rpw));
    const int64_t target = t < 1.0 ? 1 : (t >= 9.2e18 ? INT64_MAX : (int64_t)t);
    build_runs(items, cost, n, idx, target, items_out, cost_out, n_out);
    if ((rc = lpt_plan(cost_out, *n_out, n_workers, nullptr, order, worker_off, load))) return rc;
    int64_t mx = 0;
    for (int32_t w = 0; w < n_workers; ++w) mx = std::max(mx, load[w]);
    const double mean = (double)total / (double)n_workers;
    if (rpw >= max_runs_per_worker || mean == 0.0 || (double)mx / mean - 1.0 <= max_imbalance) break;
    if (*n_out == n) {
      // Every run is a single chunk: a smaller target merges nothing either,
      // so each remaining step would return this same plan.
      rpw = max_runs_per_worker;
      break;
    }
    rpw = std::min(2.0 * rpw, max_runs_per_worker);
  }
  *rpw_used = rpw;
  clear_error();
  return SKV_OK;
}
