// Internal helpers shared by the host-side translation units of libsplitkv.
#pragma once
#include <cstdarg>
#include <cstdint>

#include "splitkv.h"

namespace skv {

// Records a formatted message as the thread's last error and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

constexpr float kLog2e_host = 1.4426950408889634f;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partials of a sequence with n context keys: its chunks, plus the own-block
// partial under SKV_MASK_OWN_BLOCK.
inline int64_t n_partials(const skv_problem* p, int64_t n) {
  return ceil_div(n, p->chunk) + (p->mask == SKV_MASK_OWN_BLOCK ? 1 : 0);
}
// e_b = min(a_b + shift, N): shift is block under the prefix mask, 0 under the own-block mask.
inline int32_t end_shift(const skv_problem* p) { return p->mask == SKV_MASK_OWN_BLOCK ? 0 : p->block; }

// Per-sequence view of a validated problem (host copies).
struct SeqView {
  int64_t q0, mq, k0, n, blk0, n_blk;
};
inline SeqView seq_view(const skv_problem* p, int s) {
  SeqView v;
  v.q0 = p->h_q_off[s];
  v.mq = p->h_q_off[s + 1] - v.q0;
  v.k0 = p->h_kv_off[s];
  v.n = p->h_kv_off[s + 1] - v.k0;
  v.blk0 = v.q0 / p->block;
  v.n_blk = v.mq / p->block;
  return v;
}

}  // namespace skv
