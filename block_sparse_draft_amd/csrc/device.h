// Device-side building blocks for the gfx950 (CDNA4) kernels of libsplitkv:
// vector types, bf16 conversion, the bf16 MFMA and the LDS transpose read.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 on a 64-lane wave (lane l,
// h = l / 32):  A (32 x 16, M x K): row l % 32, k = 8h .. 8h+7;
// B (16 x 32, K x N): column l % 32, k = 8h .. 8h+7;
// C/D (32 x 32): column l % 32, element 4i + j holds row 8i + 4h + j.
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives,
// for j = 0..3, the 16-bit element i % 4 of the 8-byte chunk addressed by lane
// 4j + i / 4.  If lane 4j + q of the group addresses row r0 + j, column
// c0 + 4q of a row-major bf16 tile, lane i receives column c0 + i of rows
// r0 .. r0+3: a 4 x 16 tile read transposed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 lds_load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// 32-bit LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p);
}

// Two transposed 4 x 16 reads (see the header comment) joined into one MFMA operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// The same from 32-bit LDS byte addresses, so that constant offsets fold into
// the instructions' immediate offset fields.
__device__ __forceinline__ bf16x8 lds_tr_pair(uint32_t a0, uint32_t a1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Raw buffer descriptor over `bytes` bytes from p: loads whose offset reaches
// past the range return zeros.  Word 3 is the gfx9 raw-buffer format.  Only
// the per-lane offset may carry the position (the scalar offset of a buffer
// load is not part of the range check), so every load passes soffset = 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// A value the caller knows to be the same in every lane, moved to a scalar
// register (the compiler cannot always prove it, e.g. for fields of a work
// item loaded through a vector load).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ const T* uniform(const T* p) {
  return reinterpret_cast<const T*>(uniform(reinterpret_cast<int64_t>(p)));
}
__device__ __forceinline__ uint4 buffer_load_b128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buffer_load_b64(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// 16-byte LDS read from a 32-bit LDS byte address.
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  typedef __attribute__((address_space(3))) const uint4 lds_u4;
  return __builtin_bit_cast(bf16x8, *(lds_u4*)(uintptr_t)addr);
}

// Round-to-nearest-even fp32 -> bf16 of 8 consecutive values.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                            float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Round-to-nearest-even fp32 -> bf16 of two values, packed into one register
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a; r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// v_permlane32_swap: lanes 32..63 of `lo` trade places with lanes 0..31 of
// `hi` (lanes 0..31 of lo and 32..63 of hi keep their values).  Every lane of
// the wave must execute it.
__device__ __forceinline__ void swap_lane_halves(uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
  lo = r[0];
  hi = r[1];
}

// max(x, x of lane ^ 32) in every lane, without an LDS permute: after the swap
// lane l < 32 holds x[l] and x[l + 32] in its two registers, lane l >= 32
// x[l - 32] and x[l].
__device__ __forceinline__ float max_lane_halves(float x) {
  uint32_t a = __float_as_uint(x), b = a;
  swap_lane_halves(a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float sum_lane_halves(float x) {
  uint32_t a = __float_as_uint(x), b = a;
  swap_lane_halves(a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// max(a, b, c) as one v_max3_f32 (the compiler otherwise pairs plain v_max
// ahead of each v_max3); not volatile, so it schedules like any VALU op.  For
// kernels built without IEEE mode (no NaN quieting).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

// Worker index of this workgroup.  Workgroups are dispatched to the 8 XCDs
// round-robin, so consecutive plan workers (consecutive items of one chunk
// under LPT) are mapped to workgroups of the same XCD and share its L2.
__device__ __forceinline__ int plan_worker() {
  const int b = blockIdx.x, w = gridDim.x;
  return (w & 7) == 0 ? (b & 7) * (w >> 3) + (b >> 3) : b;
}

// Next plan slot for this workgroup, or -1 when its work is done.  The
// workgroup first claims the items of list `victim` (its own list at start)
// through the cursor claim[victim]; with `steal`, an exhausted list moves it on
// to the next worker's list, otherwise it stops there.  claim[W] counts the
// items claimed so far: once it reaches the plan's item count, no list holds
// work, so a stealing workgroup stops after one atomic instead of visiting
// every remaining list.  Uniform across the workgroup (contains barriers).
__device__ __forceinline__ int64_t claim_next(const int64_t* worker_off, int32_t* claim, int& victim, int& visited,
                                              int* s_claim, bool steal) {
  const int W = gridDim.x;
  const int lists = steal ? W : 1;
  while (visited < lists) {
    const int64_t base = worker_off[victim];
    const int64_t len = worker_off[victim + 1] - base;
    if (threadIdx.x == 0) {
      int idx = atomicAdd(&claim[victim], 1);
      if (idx < len) {
        atomicAdd(&claim[W], 1);  // one more item claimed
      } else if (steal) {
        // -1 once every item of every list is claimed
        const int seen = __hip_atomic_load(&claim[W], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen >= (int)worker_off[W]) idx = -1;
      }
      *s_claim = idx;
    }
    __syncthreads();
    // Uniform by construction; readfirstlane lets the compiler keep the item
    // and everything derived from it in scalar registers.
    const int idx = __builtin_amdgcn_readfirstlane(*s_claim);
    __syncthreads();
    if (idx < 0) return -1;
    if (idx < len) return base + idx;
    victim = victim + 1 == W ? 0 : victim + 1;
    ++visited;
  }
  return -1;
}

// Busy time of a workgroup in s_memrealtime ticks (100 MHz), written by its
// first thread to ticks[worker] when `ticks` is not NULL.
__device__ __forceinline__ void record_ticks(int64_t* ticks, int worker, uint64_t t_start) {
  if (ticks && threadIdx.x == 0) ticks[worker] = (int64_t)(__builtin_amdgcn_s_memrealtime() - t_start);
}

}  // namespace skv
