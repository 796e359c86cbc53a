// Internal helpers shared by the HIP sources of the EAGLE tree-verification library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/eagle.h"

namespace eagle {

typedef uint16_t bf16;  // IEEE bfloat16 bit pattern

// Vector types for the gfx950 bf16 MFMA builtins.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16 h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Order-preserving map float -> uint32 (larger float -> larger key; -0 < +0).
__device__ __forceinline__ uint32_t f2ord(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// 64-bit argmax key: value in the high word, (~index) in the low word, so the
// unsigned maximum is the largest value and, among equal values, the lowest index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  return ((unsigned long long)f2ord(v) << 32) | (unsigned long long)(0xffffffffu - idx);
}

// Top-k keys as doubles: the 52 mantissa bits hold (order-preserving bits of the fp32 value)
// << 20 | (2^20 - 1 - column), and the exponent field is 1, so every key is a positive
// normal double and doubles compare exactly like the packed integers (larger value first,
// then smaller column).  A compare-and-swap step of the sorted insertion is then one
// v_max_f64 and one v_min_f64 (inline: in IEEE mode the compiler would otherwise add a
// quieting max per operand).  0.0 sorts below every key and marks an empty slot.
__device__ __forceinline__ double topk_key(float v, uint32_t col) {
  const unsigned long long k = (((unsigned long long)f2ord(v) << 20) | (unsigned long long)(0xfffffu - col)) +
                               (1ull << 52);
  return __longlong_as_double((long long)k);
}
__device__ __forceinline__ float topk_key_value(unsigned long long bits) {
  return ord2f((uint32_t)((bits - (1ull << 52)) >> 20));
}
__device__ __forceinline__ int32_t topk_key_col(unsigned long long bits) {
  return (int32_t)(0xfffffu - (uint32_t)((bits - (1ull << 52)) & 0xfffffull));
}
// l = max(k, l), k = min(k, l) (l is updated in place)
__device__ __forceinline__ void topk_cas(double& k, double& l) {
  double lo;
  asm("v_min_f64 %1, %2, %0\n\tv_max_f64 %0, %2, %0" : "+v"(l), "=&v"(lo) : "v"(k));
  k = lo;
}

// Maximum of a top-k key over the 64 lanes of the wave, in the VALU only (no LDS round
// trips): DPP quad swaps (xor 1, xor 2), the half-row and row mirrors (combining the
// quads of each 8- and 16-lane row), then the 16- and 32-lane swaps of gfx950.  Every
// lane ends with the maximum.
__device__ __forceinline__ double wave_max_key(double x) {
  auto step = [](double v, double w) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(v), "v"(w));
    return r;
  };
  auto dpp = [](double v, auto ctrl) -> double {
    constexpr int C = decltype(ctrl)::value;
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, C, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), C, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  };
  x = step(x, dpp(x, std::integral_constant<int, 0xb1>{}));   // quad_perm [1,0,3,2]
  x = step(x, dpp(x, std::integral_constant<int, 0x4e>{}));   // quad_perm [2,3,0,1]
  x = step(x, dpp(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  x = step(x, dpp(x, std::integral_constant<int, 0x140>{}));  // row_mirror
  {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    x = step(__longlong_as_double((long long)(((unsigned long long)h[0] << 32) | l[0])),
             __longlong_as_double((long long)(((unsigned long long)h[1] << 32) | l[1])));
  }
  {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    x = step(__longlong_as_double((long long)(((unsigned long long)h[0] << 32) | l[0])),
             __longlong_as_double((long long)(((unsigned long long)h[1] << 32) | l[1])));
  }
  return x;
}

// Cross-workgroup hand-off without whole-cache maintenance: data meant for another
// workgroup (which may run on another XCD, with its own L2) is written and read with
// relaxed device-scope atomic accesses (global_store/load ... sc1: coherent at device
// scope), and the writer waits for its stores to complete before bumping the
// device-scope counter.  A device-scope release/acquire fence would instead write back
// and invalidate the whole L2 of the XCD (buffer_wbl2 / buffer_inv), which costs far
// more than the few kilobytes exchanged here.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until every memory operation this thread issued has completed
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// N independent sums over aligned groups of W lanes (W a power of two, <= 64), every lane
// of a group ending with its group's sum.  The shuffle distance is the outer loop, so each
// round issues the shuffles of all N values before waiting for any of them.
template <int N, int W>
__device__ __forceinline__ void group_sum_n(float (&v)[N]) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) {
    float t[N];
#pragma unroll
    for (int j = 0; j < N; ++j) t[j] = __shfl_xor(v[j], o, 64);
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] += t[j];
  }
}

// Cache addressing shared by every kernel that reads or writes a KV cache: contiguous
// (table == nullptr: b*cb + h*ch + t*ct) or paged (the page table[b*maxb + t/ps], then
// page*cb + h*ch + (t%ps)*ct; cb is the page stride).  Elements, not bytes.
struct CacheView {
  int64_t cb, ch, ct;
  const int32_t* table;
  int ps, maxb, npages;
};
// Offset of (b, h, t); a page id outside [0, npages) gives ok = false and the offset of
// a valid page (so a read stays in bounds; writers must skip the row).
__device__ __forceinline__ int64_t cache_offset(const CacheView& c, int b, int h, int t, bool& ok) {
  ok = true;
  if (!c.table) return (int64_t)b * c.cb + (int64_t)h * c.ch + (int64_t)t * c.ct;
  int pg = c.table[(int64_t)b * c.maxb + t / c.ps];
  if (pg < 0 || pg >= c.npages) {
    ok = false;
    pg = pg < 0 ? 0 : c.npages - 1;
  }
  return (int64_t)pg * c.cb + (int64_t)h * c.ch + (int64_t)(t % c.ps) * c.ct;
}

// Host: argument check of a cache layout whose element size divides 16 bytes into 8
// elements or fewer (strides in multiples of 8 elements keep every 16-byte access
// aligned for bf16 and f32 alike), and the paging fields when a block table is given.
inline int check_cache_layout(const eagle_cache_layout* c) {
  if (!c) return EAGLE_ERR_ARG;
  if (c->token_stride % 8 || c->head_stride % 8 || c->batch_stride % 8 || c->capacity < 0) return EAGLE_ERR_ARG;
  if (c->block_table) {
    if (c->page_size <= 0 || c->page_size % 64 || c->max_blocks <= 0 || c->n_pages <= 0) return EAGLE_ERR_ARG;
    if ((int64_t)c->capacity > (int64_t)c->max_blocks * c->page_size) return EAGLE_ERR_ARG;
  }
  return EAGLE_OK;
}
inline CacheView cache_view(const eagle_cache_layout* c) {
  return CacheView{c->batch_stride, c->head_stride, c->token_stride, c->block_table,
                   c->block_table ? c->page_size : 1, c->max_blocks, c->n_pages};
}

// Per-launch HIP event timing (optional).
struct Timer;
void timer_begin(eagle_timer* t, int stage, hipStream_t s);
void timer_end(eagle_timer* t, hipStream_t s);

enum Stage {
  ST_TREE_BUILD = 0, ST_QKV = 1, ST_ATTN = 2, ST_ATTN_MERGE = 3, ST_O = 4, ST_GATE_UP = 5, ST_DOWN = 6,
  ST_LM_HEAD = 7, ST_ACCEPT = 8, ST_DRAFT_FC = 9, ST_DRAFT_TOPK = 10, ST_DRAFT_SELECT = 11, ST_OTHER = 12
};

}  // namespace eagle

#define EAGLE_HIP_CHECK(expr)                         \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return EAGLE_ERR_HIP;       \
  } while (0)
