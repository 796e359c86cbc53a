// Skinny GEMM for the projections of the verify and draft paths (gfx950).
//
//   Y[m][n] = sum_k X[m][k] W[n][k],  W row-major [n][k] (bf16), X small (m <= a few hundred).
//
// With tens of token rows the projections are bound by streaming W from HBM (60 flop per
// weight byte at m = 60), so the kernel is organised around the weight stream:
//  * each workgroup owns a tile of weight rows (64..512) and a range of K; every wave
//    streams 16-row blocks of W straight from HBM into MFMA A-operand registers with
//    16-byte loads (lane l reads row l%16, 8 consecutive k), PD steps ahead;
//  * the activations (<= 64 rows per tile) are staged through LDS in K-chunks, already
//    converted to bf16 (optionally times an RMSNorm gain, with the row sum of squares
//    accumulated on the fly so the norm becomes a per-row scale in the epilogue);
//  * v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16 tokens;
//  * K is split across workgroups when the weight tiles alone cannot fill 256 CUs; the
//    last workgroup of a tile (atomic counter) sums the fp32 partials in split order,
//    so results are deterministic;
//  * the finished fp32 tile goes to LDS and a fused epilogue consumes it: rotary +
//    scatter of q/k/v, residual add, SiLU(gate)*up, or row argmax (packed 64-bit
//    atomicMax), so no intermediate [m][n] tensor makes an extra HBM round trip and
//    the LM-head logits are never written.
//  * blockIdx is remapped so that the workgroups sharing a weight tile (other token
//    tiles, other K splits) run on the same XCD and share its L2.
#include "gemm.h"

#include <algorithm>
#include <cmath>

namespace eagle {

namespace {

constexpr int kXcds = 8;

__device__ __forceinline__ int remap_xcd(int b, int total) {
  // Launch grids are padded to a multiple of 8; workgroup b runs on XCD b % 8.
  const int per = (total + kXcds - 1) / kXcds;
  return (b % kXcds) * per + b / kXcds;
}

__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  return dtype == EAGLE_BF16 ? bf2f(((const bf16*)p)[i]) : ((const float*)p)[i];
}

// Load 8 consecutive elements of X row m starting at k (k multiple of 8); returns raw
// values (before gain) in v[8].
__device__ __forceinline__ void load_x8(const XSrc& x, int m, int k, float v[8]) {
  const XSeg& sg = (k < x.ka) ? x.a : x.b;
  const int kk = (k < x.ka) ? k : k - x.ka;
  const int64_t row = sg.idx ? (int64_t)sg.idx[m] : (int64_t)m;
  if (sg.dtype == EAGLE_BF16) {
    const uint4 u = *(const uint4*)((const bf16*)sg.ptr + row * sg.ld + kk);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = (const float4*)((const float*)sg.ptr + row * sg.ld + kk);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ void apply_gain8(const XSrc& x, int k, float v[8]) {
  if (!x.gain) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= load_elem(x.gain, x.gain_dtype, k + i);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ void store_out(void* p, int dtype, int64_t i, float v) {
  if (dtype == EAGLE_BF16)
    ((bf16*)p)[i] = f2bf(v);
  else
    ((float*)p)[i] = v;
}

// Rotary inverse frequency theta^(-2j/hd) in fp64.
__device__ __forceinline__ double rope_inv_freq(int j, int hd, float theta) {
  return exp2(-(2.0 * j / hd) * log2((double)theta));
}
// Rotary angle pos * inv_freq: built in fp64 and reduced to [-pi, pi] before the fp32
// sincos, so positions up to 10^5 keep full fp32 accuracy.
__device__ __forceinline__ void rope_cs(int pos, double inv, float* c, float* s) {
  const double a = (double)pos * inv;
  const double twopi = 6.283185307179586476925286766559;
  const double r = a - rint(a * (1.0 / twopi)) * twopi;
  sincosf((float)r, s, c);
}

// EPI_STORE_F32 / EPI_RESID over a finished tile (tc <= 64 * CPL columns): token-major, a
// wave per token row and lanes along the columns (coalesced stores); the row's sum of
// squares over this tile is a wave reduction.  A wave takes U consecutive rows at a time
// and issues all their residual loads (U * CPL per lane) before any use, so one round trip
// covers them.  Every load is unconditional (RT is the residual's element type; with no
// residual, gain or row map the loads read a stand-in address inside the output and a
// select drops the value): a load under a branch would be waited for at the join.
template <int CPL, int U, typename RT>
__device__ __forceinline__ void epi_store_rows(const GemmDesc& d, const float* tile, int ts, int tc, int col0, int m0,
                                               int mv, const float* scale) {
  const Epi& e = d.epi;
  const int nw = blockDim.x / 64, w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int tile_i = col0 / tc;
  const bool has_res = e.kind == EPI_RESID && e.resid;
  const bool has_idx = has_res && e.resid_idx;
  const bool has_gain = e.xn_out && e.xn_gain;
  const RT* rp = has_res ? (const RT*)e.resid : (const RT*)e.out;
  const int64_t rld = has_res ? e.ld_resid : e.ld_out;
  const int32_t* ip = has_idx ? e.resid_idx : (const int32_t*)e.out;
  const bf16* gp = has_gain ? (const bf16*)e.xn_gain : (const bf16*)e.out;
  float gv[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = min(col0 + lane + 64 * q, d.n - 1);
    const float g = bf2f(gp[c]);
    gv[q] = has_gain ? g : 1.f;
  }
  for (int t0 = w * U; t0 < mv; t0 += nw * U) {
    int64_t rrow[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int m = m0 + min(t0 + u, mv - 1);
      const int32_t im = ip[m];
      rrow[u] = has_idx ? (int64_t)im : (int64_t)m;
    }
    float rv[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int c = min(col0 + lane + 64 * q, d.n - 1);
        const RT v = rp[rrow[u] * rld + c];
        float f;
        if constexpr (sizeof(RT) == 2) f = bf2f(v); else f = v;
        rv[u][q] = has_res ? f : 0.f;
      }
    float ss[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u;
      ss[u] = 0.f;
      if (t >= mv) continue;
      const int m = m0 + t;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int r = lane + 64 * q;
        const int c = col0 + r;
        if (r < tc && c < d.n) {
          const float v = scale[t] * tile[r * ts + t] + rv[u][q];
          e.out[(int64_t)m * e.ld_out + c] = v;
          ss[u] += v * v;
          if (e.xn_out) ((bf16*)e.xn_out)[(int64_t)m * e.ld_out + c] = f2bf(gv[q] * v);
        }
      }
    }
    if (e.ssq_out) {
      group_sum_n<U, 64>(ss);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (lane == 0 && t0 + u < mv) e.ssq_out[(int64_t)tile_i * d.m + m0 + t0 + u] = ss[u];
    }
  }
}

// EPI_TOPK with per-thread candidate lists of KL entries (KL >= k): the branch-free sorted
// insertion costs KL compare-and-swap steps per column, so the list is no longer than needed.
template <int KL>
__device__ __forceinline__ void epi_topk(const GemmDesc& d, const float* tile, int ts, int tc, int col0, int m0, int mv,
                                         int mt, const float* scale) {
  const Epi& e = d.epi;
  const int tid = threadIdx.x, nth = blockDim.x;
  // Per token: this tile's top-k (value desc, index asc) and (max, sum exp(v - max)).
  // Thread (token t = tid % mt, part = tid / mt) scans columns part, part + P, ...
  // (P = nth / mt parts per token): a wave reads one column for 64 consecutive tokens,
  // which is conflict-free in the column-major tile.  Each thread keeps its best
  // candidates as a sorted register list (branch-free insertion, static indices); the
  // partial (max, sum) pairs of a token and the lists of its parts then meet through LDS,
  // where the first part merges the others into its own list.
  const int K = e.topk;
  const int tile_i = col0 / tc;
  const int P = nth / mt;  // parts per token; threads past P * mt (mt not dividing nth) sit out
  const int t = tid % mt, part = tid / mt;
  const bool active = part < P;
  const int ncol = min(tc, d.n - col0);
  double lst[KL];
#pragma unroll
  for (int q = 0; q < KL; ++q) lst[q] = 0.0;
  float mx = -INFINITY, se = 0.f;
  if (active && t < mv) {
    const float sc = scale[t];
    int r0 = part;
    for (; r0 + 3 * P < ncol; r0 += 4 * P) {  // 4 LDS reads in flight per round
      float v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = tile[(r0 + u * P) * ts + t];
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = fmaxf(mx, sc * v4[u]);
    }
    for (; r0 < ncol; r0 += P) mx = fmaxf(mx, sc * tile[r0 * ts + t]);
    for (int r = part; r < ncol; r += P) {
      const float v = sc * tile[r * ts + t];
      se += __expf(v - mx);
      double key = topk_key(v, (uint32_t)(col0 + r));
#pragma unroll
      for (int q = 0; q < KL; ++q) topk_cas(key, lst[q]);
    }
  }
  __syncthreads();  // every read of the tile is done: its LDS is reused below
  // lists token-minor, [P][KL][mt]: the lanes of a wave (consecutive tokens) store and
  // read consecutive 8-byte words, and since mt * 2 words is a multiple of the 64 banks
  // the merge's reads stay conflict-free whatever list position each lane is at
  unsigned long long* sl = (unsigned long long*)tile;
  float* sm = (float*)(sl + (size_t)P * mt * KL);             // [P][mt][2]
  if (active) {
    if (part > 0 || P > 4) {  // (with P <= 4 part 0 keeps its list in registers)
#pragma unroll
      for (int q = 0; q < KL; ++q)
        sl[((size_t)part * KL + q) * mt + t] = (unsigned long long)__double_as_longlong(lst[q]);
    }
    sm[(part * mt + t) * 2] = mx;
    sm[(part * mt + t) * 2 + 1] = se;
  }
  __syncthreads();
  if (part == 0 && t < mv) {
    float M = -INFINITY;
    for (int p2 = 0; p2 < P; ++p2) M = fmaxf(M, sm[(p2 * mt + t) * 2]);
    float S = 0.f;
    for (int p2 = 0; p2 < P; ++p2) {
      const float m2 = sm[(p2 * mt + t) * 2];
      if (m2 > -INFINITY) S += sm[(p2 * mt + t) * 2 + 1] * __expf(m2 - M);
    }
    const int64_t ob = (int64_t)(m0 + t) * e.n_part + tile_i;  // row-major: a row's tiles adjacent
    e.lse_part[ob * 2] = M;
    e.lse_part[ob * 2 + 1] = S;
    if (P <= 4) {
      // part 0 inserts the other parts' candidates into its own register list (KL
      // compare-and-swap steps each, no LDS round trip between them)
      for (int p2 = 1; p2 < P; ++p2)
        for (int q = 0; q < KL; ++q) {
          double key = __longlong_as_double((long long)sl[((size_t)p2 * KL + q) * mt + t]);
#pragma unroll
          for (int i = 0; i < KL; ++i) topk_cas(key, lst[i]);
        }
#pragma unroll
      for (int q = 0; q < KL; ++q) {
        if (q >= K) break;
        const unsigned long long best = (unsigned long long)__double_as_longlong(lst[q]);
        const bool valid = best != 0ull;
        e.topk_val[ob * K + q] = valid ? topk_key_value(best) : -INFINITY;
        e.topk_idx[ob * K + q] = valid ? topk_key_col(best) : -1;
      }
      return;
    }
    // P-way merge of the sorted lists (keys are unique: one per column).  The heads of a
    // round are read unconditionally (clamped list and position, dropped by a select), so
    // a round costs one LDS round trip rather than one per list.
    int head[8];
#pragma unroll
    for (int p2 = 0; p2 < 8; ++p2) head[p2] = 0;
    for (int q = 0; q < K; ++q) {
      unsigned long long c[8];
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        c[p2] = sl[((size_t)min(p2, P - 1) * KL + min(head[p2], KL - 1)) * mt + t];
      if (P > 4) {
#pragma unroll
        for (int p2 = 4; p2 < 8; ++p2)
          c[p2] = sl[((size_t)min(p2, P - 1) * KL + min(head[p2], KL - 1)) * mt + t];
      } else {
#pragma unroll
        for (int p2 = 4; p2 < 8; ++p2) c[p2] = 0ull;
      }
      unsigned long long best = 0ull;
      int bp = 0;
#pragma unroll
      for (int p2 = 0; p2 < 8; ++p2) {
        const unsigned long long v = (p2 < P && head[p2] < KL) ? c[p2] : 0ull;
        if (v > best) {
          best = v;
          bp = p2;
        }
      }
#pragma unroll
      for (int p2 = 0; p2 < 8; ++p2) head[p2] += (p2 == bp && best != 0ull);
      const bool valid = best != 0ull;
      e.topk_val[ob * K + q] = valid ? topk_key_value(best) : -INFINITY;
      e.topk_idx[ob * K + q] = valid ? topk_key_col(best) : -1;
    }
  }
}

// Sampling epilogue (EPI_SAMPLE).  First the tempered logits of the child tokens that
// fall in this tile are read out and masked (sibling tokens are distinct, so every
// thread touches its own tile entries); then thread (token t = tid % mt, part = tid / mt)
// summarises its columns part, part + P, ... of the remaining logits as (max,
// sum exp(v - max)) and the largest key of v + noise.  The noise reads go out in
// batches of NQ before any is used; the per-part results are merged through LDS.
__device__ __forceinline__ void epi_sample(const GemmDesc& d, float* tile, int ts, int tc, int col0, int m0, int mv,
                                           int mt, const float* scale) {
  constexpr int NQ = 32;
  const Epi& e = d.epi;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int ncol = min(tc, d.n - col0);
  // children of rows m0 .. m0 + mv - 1 are among rows m0 + 1 .. m0 + mv + max_nodes - 2
  const int c_end = min(d.m, m0 + mv + e.max_nodes - 1);
  for (int c = m0 + 1 + tid; c < c_end; c += nth) {
    const int gp = e.gparent[c] - m0;
    const int tk = e.ctoken[c] - col0;
    if (gp >= 0 && gp < mv && tk >= 0 && tk < ncol) {
      float* at = tile + tk * ts + gp;
      e.child_logit[c] = (scale[gp] * e.inv_t) * *at;
      *at = -INFINITY;
    }
  }
  __syncthreads();
  const int tile_i = col0 / tc;
  const int P = nth / mt;  // parts per token; threads past P * mt sit out
  const int t = tid % mt, part = tid / mt;
  const bool active = part < P && t < mv;
  float mx = -INFINITY, se = 0.f;
  unsigned long long best = 0ull;
  if (active) {
    const float sc = scale[t] * e.inv_t;
    const int grp = e.row_group[m0 + t];
    const float* nz = e.noise + (int64_t)(grp < 0 ? 0 : grp) * e.ld_noise + col0;
    int r0 = part;
    for (; r0 + 3 * P < ncol; r0 += 4 * P) {
      float v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = tile[(r0 + u * P) * ts + t];
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = fmaxf(mx, sc * v4[u]);
    }
    for (; r0 < ncol; r0 += P) mx = fmaxf(mx, sc * tile[r0 * ts + t]);
    const float mref = mx == -INFINITY ? 0.f : mx;  // a part whose columns are all masked adds 0
    for (int base = part; base < ncol; base += NQ * P) {
      float g[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) g[q] = nz[min(base + q * P, ncol - 1)];  // in-range stand-in past the end
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int r = base + q * P;
        const bool in = r < ncol;
        const int rc = in ? r : ncol - 1;
        const float v = sc * tile[rc * ts + t];
        se += in ? __expf(v - mref) : 0.f;
        const unsigned long long key = in ? argmax_key(v + g[q], (uint32_t)(col0 + r)) : 0ull;
        best = key > best ? key : best;
      }
    }
  }
  __syncthreads();  // every read of the tile is done: its LDS is reused below
  float* s_mx = tile;                          // [P][mt] each
  float* s_se = s_mx + P * mt;
  uint32_t* s_klo = (uint32_t*)(s_se + P * mt);
  uint32_t* s_khi = s_klo + P * mt;
  if (part < P) {
    s_mx[part * mt + t] = mx;
    s_se[part * mt + t] = se;
    s_klo[part * mt + t] = (uint32_t)best;
    s_khi[part * mt + t] = (uint32_t)(best >> 32);
  }
  __syncthreads();
  if (part == 0 && t < mv) {
    float M = -INFINITY;
    unsigned long long K = 0ull;
    for (int p2 = 0; p2 < P; ++p2) {
      M = fmaxf(M, s_mx[p2 * mt + t]);
      const unsigned long long k2 =
          ((unsigned long long)s_khi[p2 * mt + t] << 32) | (unsigned long long)s_klo[p2 * mt + t];
      K = k2 > K ? k2 : K;
    }
    float S = 0.f;
    for (int p2 = 0; p2 < P; ++p2) {
      const float m2 = s_mx[p2 * mt + t];
      if (m2 > -INFINITY) S += s_se[p2 * mt + t] * __expf(m2 - M);
    }
    e.samp_part[(int64_t)(m0 + t) * e.n_part + tile_i] =
        make_float4(M, S, __uint_as_float((uint32_t)K), __uint_as_float((uint32_t)(K >> 32)));
  }
}

// Row argmax, after this workgroup's atomicMax of its keys: the last workgroup of the launch
// (n_epi of them) unpacks the keys and clears them (keys are only touched by device-scope
// atomics, so no cache maintenance is needed).
__device__ __forceinline__ void argmax_finish(const GemmDesc& d, int* s_flag, int n_epi) {
  const Epi& e = d.epi;
  const int tid = threadIdx.x, nth = blockDim.x;
  wait_memory();
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(e.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old == n_epi - 1);
  }
  __syncthreads();
  if (*s_flag) {
    for (int m = tid; m < d.m; m += nth) {
      const unsigned long long key = __hip_atomic_load(&e.keys[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      e.argmax_out[m] = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
      if (e.max_out) e.max_out[m] = ord2f((uint32_t)(key >> 32));
      __hip_atomic_store(&e.keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(e.done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Fused epilogue over a finished fp32 tile in LDS: tile[r * ts + t] is output column
// col0 + r (for dual tiles: gate columns r < tc, up columns r >= tc) of token m0 + t,
// before the per-row norm scale scale[t].
// CPLC: output columns per lane of the store epilogue, ceil(tc / 64) at most.
template <int CPLC, bool WITH_SAMPLE, bool WITH_TOPK = true>
__device__ void run_epilogue(const GemmDesc& d, const float* tile, int ts, int tc, int col0, int m0, int mv,
                             int mt, const float* scale, float* red_scratch, int* s_flag, int n_epi) {
  const Epi& e = d.epi;
  const int tid = threadIdx.x, nth = blockDim.x;
  switch (e.kind) {
    case EPI_STORE_F32:
    case EPI_RESID: {
      constexpr int U = CPLC >= 16 ? 1 : 16 / CPLC;
      if (e.kind == EPI_RESID && e.resid && e.resid_dtype == EAGLE_BF16)
        epi_store_rows<CPLC, U, bf16>(d, tile, ts, tc, col0, m0, mv, scale);
      else
        epi_store_rows<CPLC, U, float>(d, tile, ts, tc, col0, m0, mv, scale);
      break;
    }
    case EPI_SILU: {
      for (int i = tid; i < tc * mv; i += nth) {
        const int r = i % tc, t = i / tc;
        const int c = col0 + r;
        if (c >= d.n) continue;
        const float g = scale[t] * tile[r * ts + t];
        const float u = scale[t] * tile[(tc + r) * ts + t];
        store_out(e.act, e.act_dtype, (int64_t)(m0 + t) * e.ld_act + c, silu(g) * u);
      }
      break;
    }
    case EPI_QKV: {
      __shared__ int s_pos[256], s_kvrow[256];  // token tiles hold at most 256 rows
      for (int t = tid; t < mv; t += nth) {
        s_pos[t] = e.pos ? e.pos[m0 + t] : 0;
        s_kvrow[t] = e.kv_idx ? e.kv_idx[m0 + t] : m0 + t;
      }
      __syncthreads();
      const int hd = e.hd, half = hd / 2;
      const int heads_in_tile = tc / hd;
      // nth is a multiple of half, so every thread keeps the same pair index j
      const int j = tid % half;
      const double inv = e.theta > 0.f ? rope_inv_freq(j, hd, e.theta) : 0.0;
      for (int i = tid; i < mv * heads_in_tile * half; i += nth) {
        const int hl = (i / half) % heads_in_tile;
        const int t = i / (half * heads_in_tile);
        const int head = col0 / hd + hl;
        if (head >= e.hq + 2 * e.hkv) continue;
        const int m = m0 + t;
        float a = scale[t] * tile[(hl * hd + j) * ts + t];
        float b = scale[t] * tile[(hl * hd + j + half) * ts + t];
        if (head < e.hq + e.hkv && e.theta > 0.f) {
          float c, s;
          rope_cs(s_pos[t], inv, &c, &s);
          const float ra = a * c - b * s;
          const float rb = b * c + a * s;
          a = ra;
          b = rb;
        }
        void* dst;
        int64_t base;
        if (head < e.hq) {
          dst = e.q_out;
          base = ((int64_t)m * e.hq + head) * hd;
        } else if (head < e.hq + e.hkv) {
          if (s_kvrow[t] < 0) continue;
          dst = e.k_out;
          base = ((int64_t)s_kvrow[t] * e.hkv + (head - e.hq)) * hd;
        } else {
          if (s_kvrow[t] < 0) continue;
          dst = e.v_out;
          base = ((int64_t)s_kvrow[t] * e.hkv + (head - e.hq - e.hkv)) * hd;
        }
        store_out(dst, e.out_dtype, base + j, a);
        store_out(dst, e.out_dtype, base + j + half, b);
      }
      break;
    }
    case EPI_ARGMAX: {
      // thread -> (token t, row stripe); rows are scanned in increasing order so the
      // first maximum wins, then stripes are merged through LDS with the packed key.
      const int stripes = nth / mt;  // threads past stripes * mt (mt not dividing nth) sit out
      const int t = tid % mt, st = tid / mt;
      unsigned long long best = 0ull;
      if (t < mv && st < stripes) {
        const float sc = scale[t];
        const int rlim = min(tc, d.n - col0);
        int r = st;
        if (!e.dbg_logits) {
          // 8 rows per round: the LDS reads of a round are issued before any use
          for (; r + 7 * stripes < rlim; r += 8 * stripes) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = tile[(r + u * stripes) * ts + t];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const unsigned long long key = argmax_key(sc * v[u], (uint32_t)(col0 + r + u * stripes));
              best = key > best ? key : best;
            }
          }
        }
        for (; r < rlim; r += stripes) {
          const int c = col0 + r;
          const float v = sc * tile[r * ts + t];
          if (e.dbg_logits) e.dbg_logits[(int64_t)(m0 + t) * e.ld_logits + c] = v;
          const unsigned long long key = argmax_key(v, (uint32_t)c);
          best = key > best ? key : best;
        }
      }
      unsigned long long* red = (unsigned long long*)red_scratch;
      red[tid] = best;
      __syncthreads();
      if (tid < mt && tid < mv) {
        unsigned long long b2 = red[tid];
        for (int s2 = 1; s2 < stripes; ++s2) {
          const unsigned long long o = red[s2 * mt + tid];
          b2 = o > b2 ? o : b2;
        }
        atomicMax(&e.keys[m0 + tid], b2);
      }
      argmax_finish(d, s_flag, n_epi);
      break;
    }
    case EPI_SAMPLE:
      if constexpr (WITH_SAMPLE) epi_sample(d, const_cast<float*>(tile), ts, tc, col0, m0, mv, mt, scale);
      break;
    case EPI_TOPK: {
      // (every list length is inlined into each tile instance that carries the top-k
      // epilogue: the eight-wave tiles of up to 160 tokens, which have the registers)
      if constexpr (WITH_TOPK) {
        if (e.topk <= 10)
          epi_topk<10>(d, tile, ts, tc, col0, m0, mv, mt, scale);
        else if (e.topk <= 12)
          epi_topk<12>(d, tile, ts, tc, col0, m0, mv, mt, scale);
        else
          epi_topk<16>(d, tile, ts, tc, col0, m0, mv, mt, scale);
      }
      break;
    }
    default:
      break;
  }
}

// Split-K partial tiles are exchanged in MFMA-fragment order (fragment f = (16-row block,
// 16-token block), lane l: its four accumulators as one 16-byte vector) with 16-byte
// buffer loads and stores carrying the device-coherent cache policy (SC1, the policy of
// agent-scope atomic accesses): the partials come from workgroups on other XCDs, whose L2
// is not coherent with this one.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kSc1 = 16;  // cache-policy bits of a buffer access: SC1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Epilogue halves: a tile whose fp32 output would not fit LDS runs its epilogue twice, on
// half of its weight-row blocks each time.  Block blk (of NB) belongs to half h and is
// block lb of that half's tile; for gate/up tiles each half holds matching gate and up
// column blocks (gate blocks first), so it is itself a gate/up tile of half the columns.
template <int EH, bool DUAL, int NB>
__device__ __forceinline__ int half_to_block(int h, int lb) {
  if (EH == 1) return lb;
  if (!DUAL) return h * (NB / 2) + lb;
  constexpr int Q = NB / 4;  // gate (or up) blocks per half
  return lb < Q ? h * Q + lb : NB / 2 + h * Q + (lb - Q);
}
template <int EH, bool DUAL, int NB>
__device__ __forceinline__ bool block_in_half(int blk, int h, int* lb) {
  if (EH == 1) {
    *lb = blk;
    return true;
  }
  if (!DUAL) {
    *lb = blk % (NB / 2);
    return blk / (NB / 2) == h;
  }
  constexpr int Q = NB / 4;
  const bool up = blk >= NB / 2;
  const int b2 = up ? blk - NB / 2 : blk;
  *lb = (up ? Q : 0) + b2 % Q;
  return b2 / Q == h;
}

// Split-K fixup of epilogue half h: tile = sum over splits (in split order) of the S partial
// tiles of NF4 fragments each.  All loads of a pass are issued before the first add, so
// the round trips to memory overlap.
template <int S, int NF4, int MT_, int TS_, int NTH_, int EH, bool DUAL, int NB>
__device__ __forceinline__ void sum_partials(const float* p0, float* tile, int h) {
  constexpr int NFH = NF4 / EH;  // fragments of one half
  // fragments per thread per pass: up to 32 loads of 16 bytes in flight per thread (the
  // main loop's registers are free by now), so a tile usually takes a single round trip;
  // tiles with two epilogue halves keep their accumulators live meanwhile and take 8
  constexpr int LOADS = EH == 1 ? 32 : 8;
  constexpr int GMAX = LOADS / S > 0 ? LOADS / S : 1;
  constexpr int GNEED = (NFH + NTH_ - 1) / NTH_;
  constexpr int G = GMAX < GNEED ? GMAX : GNEED;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p0, (uint32_t)S * NF4 * 16);
  for (int f0 = threadIdx.x; f0 < NFH; f0 += NTH_ * G) {
    f32x4 a[S][G];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int fl = min(f0 + g * NTH_, NFH - 1);  // fragment of the half tile
        const int bt = fl / 64;
        const int f = (half_to_block<EH, DUAL, NB>(h, bt / (MT_ / 16)) * (MT_ / 16) + bt % (MT_ / 16)) * 64 + fl % 64;
        a[s][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (s * NF4 + f) * 16, 0, kSc1));
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int fl = f0 + g * NTH_;
      if (fl >= NFH) break;
      f32x4 v = a[0][g];
#pragma unroll
      for (int s = 1; s < S; ++s) v += a[s][g];
      // fragment: 16-row block lb, 16-token block t, lane l -> rows lb*16 + (l/16)*4 + i
      const int l = fl % 64, bt = fl / 64;
      const int t = bt % (MT_ / 16), lb = bt / (MT_ / 16);
      float* dst = tile + (lb * 16 + (l / 16) * 4) * TS_ + t * 16 + (l % 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * TS_] = v[i];
    }
  }
}

// ---------------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------------
// Tile shapes: NW waves x RB 16-row weight blocks per wave, MT tokens, K chunks of KC,
// XB X-chunk buffers in LDS (1: the next chunk is stored after a barrier), EH epilogue
// halves (2: the fp32 output tile is formed and consumed one half at a time).  Wider token
// tiles (MT 128 / 256) use shorter K chunks so that the X chunks and the output tile both
// fit the 160 KB of LDS; each weight byte is then streamed once per MT tokens instead of
// once per 64.
// SAMPLE: the instance for the sampling epilogue only (the other epilogues' code and its
// registers stay out of it, and it stays out of theirs).
template <int NW, int RB, int PD, bool DUAL, int MT, int KC, int XB, int EH, bool SAMPLE>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(GemmDesc d, int grid_real) {
  constexpr int NT = NW * RB * 16;        // weight rows per tile (both blocks when DUAL)
  constexpr int TC = DUAL ? NT / 2 : NT;  // output columns per tile
  constexpr int NSTEP = KC / 32;
  constexpr int XS = KC + 8;              // LDS row stride of an X chunk (bf16)
  constexpr int TS = MT + 4;              // LDS row stride of the output tile (f32)
  constexpr int LDS_X = XB * MT * XS * 2;  // X chunk buffers
  constexpr int LDS_T = NT / EH * TS * 4;  // one epilogue half of the output tile
  constexpr int NB = NT / 16;               // 16-row weight blocks per tile
  constexpr int LDS = LDS_X > LDS_T ? LDS_X : LDS_T;
  constexpr int LPR = KC / 8;             // lanes staging one X row (16 bytes each)
  constexpr int RPP = 64 / LPR;           // X rows per wave per pass
  constexpr int RPW = MT / (NW * RPP);    // passes: X registers per thread
  constexpr int NTH = NW * 64;
  // Four-wave tiles ("wide" mode, for hundreds of token rows) run one wave per SIMD with
  // v_mfma_f32_32x32x16_bf16: a single wave keeps the matrix core busy only with the 32x32
  // shape (the 16x16 one needs two waves per SIMD), and each wave has the whole register
  // file for its accumulators.  The weight fragments stay in the 16-row layout; a lane
  // swap turns two of them into the operands of two 32-row MFMAs (below).
  constexpr bool W32 = NW == 4;
  // the top-k epilogue is compiled into the eight-wave tiles of 64 to 160 tokens only (the
  // planner never gives it the others)
  constexpr bool TOPK_TILE = !W32 && MT <= 160 && MT >= 64;
  static_assert(!W32 || (RB % 2 == 0 && MT % 32 == 0), "wide tiles pair 16-row blocks and use 32-token blocks");
  static_assert(!W32 || (XB == 2 && NSTEP >= 2 && RPW == MT / 16), "wide tiles stage one X row per MFMA group");
  static_assert(NSTEP % PD == 0, "prefetch depth must divide the chunk steps");
  static_assert(LPR <= 64 && 64 % LPR == 0 && MT % (NW * RPP) == 0, "X staging layout");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(NW * MT * 8 <= LDS, "argmax reduction buffer");
  static_assert(MT <= NTH && MT <= 256, "token tile");

  __shared__ __align__(16) unsigned char smem[LDS];
  __shared__ float s_scale[MT];
  __shared__ float s_ssq[MT];
  __shared__ unsigned long long s_red[NTH];
  __shared__ int s_flag;

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  if (bid >= grid_real) return;
  // the wave index is wave-uniform; saying so keeps per-wave row offsets in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  const int m_tiles = (d.m + MT - 1) / MT;
  int b = bid;
  const int split = b % d.splits;
  b /= d.splits;
  const int mt_i = b % m_tiles;
  const int nt_i = b / m_tiles;
  const int col0 = nt_i * TC, m0 = mt_i * MT;
  const int mv = min(MT, d.m - m0);
  const int kps = d.kps;
  const int kb = split * kps;
  const int ke = min(d.k, kb + kps);
  const int klast = ke - 32;
  // chunks of this K range, visited in a rotated order so that concurrently running
  // workgroups read different columns (spreads requests over HBM channels); the token
  // tiles of one weight tile run side by side on one XCD and keep the same order, so
  // the weight lines the first one fetches are still in that XCD's L2 for the others
  // (the same order for both weight layouts, so they give bit-identical results).  With
  // several token tiles every workgroup walks K from the start instead: the workgroups
  // resident on an XCD then read the same activation chunk at about the same time, and
  // the activations (re-read once per weight tile) come from L2 rather than from beyond it.
  const int nchunk = (ke - kb + KC - 1) / KC;
  const int c0 = m_tiles > 1 ? 0 : (nt_i * 5 + split * 3) % nchunk;

  // norm == 2: the row sums of squares arrive as np per-tile partials.  Their loads are
  // issued here, spread over all threads (part = tid / MT, 4 loads in flight per thread),
  // so the round trips hide under the main loop; the tail adds the parts in fixed order.
  constexpr int NPART = NTH / MT;
  float* s_np = (float*)s_red;  // [NPART][MT]; s_red is not used before the epilogue
  // Up to 4 partials per thread stay in registers, unsummed, until after the main loop, so
  // nothing waits for them here; more than that are summed (and waited for) right away.
  const bool np_regs = d.x.norm == 2 && d.x.np <= 4 * NPART;
  float np_a[4] = {0.f, 0.f, 0.f, 0.f};
  if (np_regs) {
    const int row = tid % MT, part = tid / MT;
    const int m = min(m0 + row, d.m - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = min(min(part, NPART - 1) + u * NPART, d.x.np - 1);
      np_a[u] = d.x.ssq_in[(int64_t)p * d.m + m];
    }
  } else if (d.x.norm == 2) {
    const int row = tid % MT, part = tid / MT;
    if (part < NPART) {
      const int m = min(m0 + row, d.m - 1);
      float v = 0.f;
      for (int p0 = part; p0 < d.x.np; p0 += 4 * NPART) {
        float a4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int p = min(p0 + u * NPART, d.x.np - 1);
          a4[u] = d.x.ssq_in[(int64_t)p * d.m + m];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) v += (p0 + u * NPART < d.x.np) ? a4[u] : 0.f;
      }
      s_np[part * MT + row] = v;
    }
  }

  // this wave's weight rows
  const bf16* wblk;
  int wrow0;
  if (DUAL) {
    constexpr int HALF = NW / 2;
    wblk = (const bf16*)((wid < HALF) ? d.w0 : d.w1);
    wrow0 = col0 + (wid % HALF) * RB * 16;
  } else {
    wblk = (const bf16*)d.w0;
    wrow0 = col0 + wid * RB * 16;
  }
  // wp[rb]: this lane's 8 elements of block rb at K step 0; wstep: elements between
  // consecutive 32-column steps (the address of column k is wp + (k / 32) * wstep)
  const bf16* wp[RB];
  int64_t wstep;
  if (d.w_layout) {
    const int nblk = (d.n + 15) / 16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) wp[rb] = wblk + (int64_t)min(wrow0 / 16 + rb, nblk - 1) * 512 + lane * 8;
    wstep = (int64_t)nblk * 512;
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = min(wrow0 + rb * 16 + lr, d.n - 1);
      wp[rb] = wblk + (int64_t)row * d.ldw + lq * 8;
    }
    wstep = 32;
  }
  // Weight loads carry the non-temporal hint: each weight line is used by this launch only
  // (and by the few token tiles of its weight tile, which run together on one XCD), so the
  // stream should not displace what the caches hold for the activations and partials.
  // Measured: the 60-row LM head 186 -> 165 us (1.05 GB at 6.4 TB/s), the 70B layer at 60
  // rows 10% faster, the draft expansion 6%; neutral at 960 rows.
  auto wload = [&](int rb, int k) {
    return __builtin_nontemporal_load((const bf16x8_t*)(wp[rb] + (int64_t)(k >> 5) * wstep));
  };

  // X rows staged by this lane: r = (wid + j * NW) * RPP + lane / LPR, 8 columns at
  // (lane % LPR) * 8 of each chunk
  const int xl_row = lane / LPR, xl_col = (lane % LPR) * 8;
  // (source row indices kept as 32-bit values: wide tiles stage many rows per thread)
  int32_t xrow_a[RPW], xrow_b[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int m = min(m0 + (wid + j * NW) * RPP + xl_row, d.m - 1);
    xrow_a[j] = d.x.a.idx ? d.x.a.idx[m] : m;
    xrow_b[j] = d.x.b.idx ? d.x.b.idx[m] : m;
  }
  auto chunk_k = [&](int ci) {
    int c = c0 + ci;
    if (c >= nchunk) c -= nchunk;
    return kb + c * KC;
  };
  uint4 xr[RPW];
  uint4 gr = make_uint4(0u, 0u, 0u, 0u);  // norm == 1: the 8 gain values of this lane's columns
  const bool stage_gain = d.x.norm == 1 && d.x.gain;
  // the gain load is unconditional (a load under a branch is waited for at the join); with
  // no gain it reads the weights (at least k elements) and the value is not used
  const bf16* gain_src = stage_gain ? (const bf16*)d.x.gain : (const bf16*)d.w0;
  auto load_x = [&](int kc) {
    const int k = min(kc + xl_col, ke - 8);  // clamped: out-of-range lanes are zeroed at store
    gr = *(const uint4*)(gain_src + k);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const bool in_a = k < d.x.ka;
      const bf16* base = in_a ? (const bf16*)d.x.a.ptr + (int64_t)xrow_a[j] * d.x.a.ld + k
                              : (const bf16*)d.x.b.ptr + (int64_t)xrow_b[j] * d.x.b.ld + (k - d.x.ka);
      xr[j] = *(const uint4*)base;
    }
  };
  float ssq[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) ssq[j] = 0.f;
  auto store_x = [&](int buf, int kc, float ssq_w) {
    bf16* xl = (bf16*)smem + buf * (MT * XS);
    const int k = kc + xl_col;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = (wid + j * NW) * RPP + xl_row;
      uint4 v = xr[j];
      if (!(m0 + r < d.m && k < ke)) v = make_uint4(0u, 0u, 0u, 0u);
      if (d.x.norm == 1) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = __uint_as_float(w4[i] << 16);
          f[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) ssq[j] += ssq_w * f[i] * f[i];
        if (stage_gain) {
          const uint32_t g4[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[2 * i] *= __uint_as_float(g4[i] << 16);
            f[2 * i + 1] *= __uint_as_float(g4[i] & 0xffff0000u);
          }
          v = make_uint4(pack2bf(f[0], f[1]), pack2bf(f[2], f[3]), pack2bf(f[4], f[5]), pack2bf(f[6], f[7]));
        }
      }
      *(uint4*)(xl + r * XS + xl_col) = v;
    }
  };

  // Wide mode stages X one row at a time, each row store and load placed between two MFMA
  // groups of a step, so the staging work overlaps the matrix core instead of stalling it.
  // The gain values of a chunk are requested after its last row store (gr then holds the
  // gain of the chunk whose rows are in flight).
  auto load_row = [&](int j, int kc) {
    const int k = min(kc + xl_col, ke - 8);
    const bool in_a = k < d.x.ka;
    const bf16* base = in_a ? (const bf16*)d.x.a.ptr + (int64_t)xrow_a[j] * d.x.a.ld + k
                            : (const bf16*)d.x.b.ptr + (int64_t)xrow_b[j] * d.x.b.ld + (k - d.x.ka);
    xr[j] = *(const uint4*)base;
  };
  auto load_gain = [&](int kc) { gr = *(const uint4*)(gain_src + min(kc + xl_col, ke - 8)); };
  auto store_row = [&](int j, int buf, int kc, float ssq_w) {
    bf16* xl = (bf16*)smem + buf * (MT * XS);
    const int r = (wid + j * NW) * RPP + xl_row;
    // rows past m and columns past the K range are zero (a mask, not a branch)
    const uint32_t keep = (m0 + r < d.m && kc + xl_col < ke) ? 0xffffffffu : 0u;
    uint4 v = make_uint4(xr[j].x & keep, xr[j].y & keep, xr[j].z & keep, xr[j].w & keep);
    if (d.x.norm == 1) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w4[i] << 16);
        f[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ssq[j] += ssq_w * f[i] * f[i];
      if (stage_gain) {
        const uint32_t g4[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] *= __uint_as_float(g4[i] << 16);
          f[2 * i + 1] *= __uint_as_float(g4[i] & 0xffff0000u);
        }
        v = make_uint4(pack2bf(f[0], f[1]), pack2bf(f[2], f[3]), pack2bf(f[4], f[5]), pack2bf(f[6], f[7]));
      }
    }
    *(uint4*)(xl + r * XS + xl_col) = v;
  };

  // (one of the two accumulator sets is used: 16x16 fragments, or 32x32 ones in wide mode)
  f32x4 acc[W32 ? 1 : RB][W32 ? 1 : MT / 16];
  f32x16 acc32[W32 ? RB / 2 : 1][W32 ? MT / 32 : 1];
#pragma unroll
  for (int rb = 0; rb < (W32 ? 1 : RB); ++rb)
#pragma unroll
    for (int t = 0; t < (W32 ? 1 : MT / 16); ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < (W32 ? RB / 2 : 1); ++p)
#pragma unroll
    for (int t = 0; t < (W32 ? MT / 32 : 1); ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc32[p][t][q] = 0.f;

  // Weight prefetch ring.  Loads are unconditional (addresses past the K range are
  // clamped to its last step): a conditional load would make the compiler wait for it
  // before merging the ring register, which serialises the stream.
  bf16x8_t wbuf[PD][RB];
  {
    // the first X chunk is requested before the weight ring: loads return in order, so
    // the chunk (and the barrier after it) waits for one round trip, not for the whole ring
    const int kc = chunk_k(0);
    load_x(kc);
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int k = min(kc + s * 32, klast);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wbuf[s][rb] = wload(rb, k);
    }
    store_x(0, kc, 1.f);
    // wide mode: the rows of the chunk after next are requested during a chunk's second
    // step (below), so the second chunk is requested here
    if (W32) {
#pragma unroll
      for (int j = 0; j < RPW; ++j) load_row(j, chunk_k(min(1, nchunk - 1)));
      load_gain(chunk_k(min(1, nchunk - 1)));
    }
  }
  __syncthreads();

  for (int ci = 0; ci < nchunk; ++ci) {
    const int kc = chunk_k(ci);
    const bool more = ci + 1 < nchunk;
    const int kcn = chunk_k(more ? ci + 1 : 0);
    // next chunk's X: issued now, stored to the other buffer after this chunk's math (wide
    // mode: stored half-way through this chunk, when the chunk after it is requested)
    if (!W32 && more) load_x(kcn);
    const bf16* xl = (const bf16*)smem + (XB == 2 ? (ci & 1) : 0) * (MT * XS);
    // Every chunk runs all NSTEP steps: past the K range X is zero in LDS, so the
    // extra steps of a short chunk add exact zeros (and stay branch-free).
    if constexpr (W32) {
      // Lane swap of a pair of 16-row fragments (rows 0-15 and 16-31 of a 32-row block;
      // lane group g of 16 lanes holds k group g of 8): the first result holds k groups 0
      // and 2 of rows 0-31 in the lane order of a 32x32x16 A operand (lane l: row l % 32,
      // k slot l / 32), the second k groups 1 and 3.  The X operand of the matching MFMA
      // reads the same k groups: lane l takes token l % 32 and k group (l / 32) * 2 + h.
      // Fragment (t, h) of the next step is read right after its last MFMA of this step.
      bf16x8_t xf[MT / 32][2];
      const bf16* xrd = xl + (lane & 31) * XS + (lane >> 5) * 16;
#pragma unroll
      for (int t = 0; t < MT / 32; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) xf[t][h] = *(const bf16x8_t*)(xrd + t * 32 * XS + h * 8);
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        int kn = (s + PD < NSTEP) ? kc + (s + PD) * 32 : (more ? kcn + (s + PD - NSTEP) * 32 : klast);
        kn = min(kn, klast);
        // The ring slot is swapped in place and refilled after the MFMAs that read it (the
        // operands of the first k half after that half's MFMAs), so every slot keeps its
        // registers from one chunk to the next.
#pragma unroll
        for (int p = 0; p < RB / 2; ++p) {
          u32x4_t lo = __builtin_bit_cast(u32x4_t, wbuf[s % PD][2 * p]);
          u32x4_t hi = __builtin_bit_cast(u32x4_t, wbuf[s % PD][2 * p + 1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(lo[i], hi[i], false, false);
            lo[i] = r[0];
            hi[i] = r[1];
          }
          wbuf[s % PD][2 * p] = __builtin_bit_cast(bf16x8_t, lo);
          wbuf[s % PD][2 * p + 1] = __builtin_bit_cast(bf16x8_t, hi);
        }
        __builtin_amdgcn_sched_barrier(0);
        // (the k halves outermost: consecutive MFMAs into one accumulator are MT / 32 * RB / 2
        // instructions apart, past the 32x32 MFMA's latency)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int t = 0; t < MT / 32; ++t) {
#pragma unroll
            for (int p = 0; p < RB / 2; ++p)
              acc32[p][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wbuf[s % PD][2 * p + h], xf[t][h], acc32[p][t], 0, 0, 0);
            if (s + 1 < NSTEP) xf[t][h] = *(const bf16x8_t*)(xrd + t * 32 * XS + (s + 1) * 32 + h * 8);
            if (s == 1) {
              // row j of the next chunk (requested a chunk ago) goes to the other buffer,
              // whose last reads were before the previous barrier; then row j of the chunk
              // after it is requested (MT / 16 groups per step, one row each; both
              // unconditional: past the last chunk they stage the last chunk again into
              // the idle buffer, and a load under a branch would be waited for at the join)
              const int j = h * (MT / 32) + t;
              const int kc2 = chunk_k(min(ci + 2, nchunk - 1));
              store_row(j, (ci + 1) & 1, kcn, more ? 1.f : 0.f);  // (no sum of squares past the end)
              load_row(j, kc2);
              if (j == RPW - 1) load_gain(kc2);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          // this half's operands are consumed: their slot registers take the weights of
          // step s + PD
#pragma unroll
          for (int p = 0; p < RB / 2; ++p) wbuf[s % PD][2 * p + h] = wload(2 * p + h, kn);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      bf16x8_t cur[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) cur[rb] = wbuf[s % PD][rb];
      int kn = (s + PD < NSTEP) ? kc + (s + PD) * 32 : (more ? kcn + (s + PD - NSTEP) * 32 : klast);
      kn = min(kn, klast);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wbuf[s % PD][rb] = wload(rb, kn);
      // keep the prefetch of step s + PD ahead of the math of step s (the scheduler
      // would otherwise sink the loads next to their use)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < MT / 16; ++t) {
        const bf16x8_t xf = *(const bf16x8_t*)(xl + (t * 16 + lr) * XS + s * 32 + lq * 8);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[rb], xf, acc[rb][t], 0, 0, 0);
      }
    }
    }
    if (W32) {
      __syncthreads();
    } else if (XB == 2) {
      if (more) store_x((ci + 1) & 1, kcn, 1.f);
      __syncthreads();
    } else {
      // one buffer: every wave is done with this chunk before it is overwritten
      __syncthreads();
      if (more) {
        store_x(0, kcn, 1.f);
        __syncthreads();
      }
    }
  }

  // row sums of squares of this K range (norm == 1): the LPR lanes of a row are adjacent
  if (d.x.norm == 1) {
    group_sum_n<RPW, LPR>(ssq);
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      if (lane % LPR == 0) s_ssq[(wid + j * NW) * RPP + xl_row] = ssq[j];
  }
  if (np_regs) {
    const int row = tid % MT, part = tid / MT;
    if (part < NPART) {
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) v += (part + u * NPART < d.x.np) ? np_a[u] : 0.f;
      s_np[part * MT + row] = v;
    }
  }
  __syncthreads();

  float* tile = (float*)smem;
  const int tile_id = nt_i * m_tiles + mt_i;
  auto row_scale = [&](float ssq_total) -> float {
    if (d.x.norm == 1) return rsqrtf(ssq_total / (float)d.k + d.x.eps);
    return 1.f;
  };
  if (d.splits > 1) {
    // split-K: publish this split's partial tile; the last split of the tile to arrive
    // sums all partials in split order (deterministic) and runs the epilogue
    float* part = d.partials + ((int64_t)tile_id * d.splits + split) * (NT * MT);
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(part, NT * MT * 4);
    // (wide tiles run with a single K split: the launch refuses anything else)
    if constexpr (!W32) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t = 0; t < MT / 16; ++t) {
          const int f = ((wid * RB + rb) * (MT / 16) + t) * 64 + lane;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[rb][t]), prs, f * 16, 0, kSc1);
        }
    }
    if (d.x.norm == 1 && tid < MT)
      coherent_store(d.sumsq_part + ((int64_t)tile_id * d.splits + split) * MT + tid, s_ssq[tid]);
    wait_memory();
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(&d.counters[tile_id], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = (old == d.splits - 1);
    }
    __syncthreads();
    if (!s_flag) return;  // another split runs this tile's epilogue
    if (d.x.norm == 1 && tid < MT) {
      float v = 0.f;
      for (int s = 0; s < d.splits; ++s) v += coherent_load(d.sumsq_part + ((int64_t)tile_id * d.splits + s) * MT + tid);
      s_ssq[tid] = v;
    }
    if (tid == 0) __hip_atomic_store(&d.counters[tile_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < MT) {
    float sc = row_scale(s_ssq[tid]);
    if (d.x.norm == 2) {
      float v = 0.f;
      for (int part = 0; part < NPART; ++part) v += s_np[part * MT + tid];
      sc = rsqrtf(v / (float)d.k + d.x.eps);
    }
    s_scale[tid] = sc;
  }
  if (d.epi.kind == EPI_ARGMAX && !d.epi.dbg_logits && d.splits == 1 && !DUAL && !SAMPLE) {
    // Row argmax straight from the accumulators: each lane keeps the best key of its
    // tokens over its own columns, the lanes holding the same token combine by cross-lane
    // swaps and the waves through LDS, and one atomicMax per token leaves the workgroup
    // (no fp32 tile in LDS, no epilogue halves).  Same keys as the tile path: the scaled
    // value of each logit and its column.
    __syncthreads();  // s_scale is ready; every wave is done with the X buffers
    unsigned long long* red = (unsigned long long*)smem;  // [NW][MT]
    if constexpr (W32) {
#pragma unroll
      for (int t = 0; t < MT / 32; ++t) {
        const float sc = s_scale[t * 32 + (lane & 31)];
        unsigned long long best = 0ull;
#pragma unroll
        for (int p = 0; p < RB / 2; ++p)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int c = col0 + wid * RB * 16 + p * 32 + 8 * (q >> 2) + (lane >> 5) * 4 + (q & 3);
            const unsigned long long key = c < d.n ? argmax_key(sc * acc32[p][t][q], (uint32_t)c) : 0ull;
            best = key > best ? key : best;
          }
        const unsigned long long o = shfl_xor_u64(best, 32);
        best = o > best ? o : best;
        if (lane < 32) red[wid * MT + t * 32 + lane] = best;
      }
    } else {
#pragma unroll
      for (int t = 0; t < MT / 16; ++t) {
        const float sc = s_scale[t * 16 + lr];
        unsigned long long best = 0ull;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = col0 + wid * RB * 16 + rb * 16 + lq * 4 + i;
            const unsigned long long key = c < d.n ? argmax_key(sc * acc[rb][t][i], (uint32_t)c) : 0ull;
            best = key > best ? key : best;
          }
        unsigned long long o = shfl_xor_u64(best, 16);
        best = o > best ? o : best;
        o = shfl_xor_u64(best, 32);
        best = o > best ? o : best;
        if (lane < 16) red[wid * MT + t * 16 + lane] = best;
      }
    }
    __syncthreads();
    if (tid < mv) {
      unsigned long long b2 = red[tid];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) {
        const unsigned long long o = red[w2 * MT + tid];
        b2 = o > b2 ? o : b2;
      }
      atomicMax(&d.epi.keys[m0 + tid], b2);
    }
    argmax_finish(d, &s_flag, ((d.n + TC - 1) / TC) * m_tiles);
    return;
  }
  constexpr int TCH = TC / EH;  // output columns of one epilogue half
  const int n_epi = ((d.n + TC - 1) / TC) * m_tiles * EH;
  for (int h = 0; h < EH; ++h) {
    if (h) __syncthreads();  // the previous half's epilogue is done with the tile
    if (d.splits == 1 && W32) {
      // 32x32 accumulators: q = 4 * qq + i is row 8 * qq + (lane / 32) * 4 + i of the pair,
      // token lane % 32; rows 0-15 belong to 16-row block 2 * p, rows 16-31 to 2 * p + 1
#pragma unroll
      for (int p = 0; p < (W32 ? RB / 2 : 1); ++p)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          int lb;
          if (!block_in_half<EH, DUAL, NB>(wid * RB + 2 * p + hb, h, &lb)) continue;  // wave-uniform
#pragma unroll
          for (int t = 0; t < (W32 ? MT / 32 : 1); ++t)
#pragma unroll
            for (int q2 = 0; q2 < 8; ++q2) {
              const int q = hb * 8 + q2;
              const int rr = 8 * (q2 / 4) + (lane >> 5) * 4 + (q2 & 3);
              tile[(lb * 16 + rr) * TS + t * 32 + (lane & 31)] = acc32[p][t][q];
            }
        }
    } else if (d.splits == 1) {
#pragma unroll
      for (int rb = 0; rb < (W32 ? 1 : RB); ++rb) {
        int lb;
        if (!block_in_half<EH, DUAL, NB>(wid * RB + rb, h, &lb)) continue;  // wave-uniform
#pragma unroll
        for (int t = 0; t < (W32 ? 1 : MT / 16); ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) tile[(lb * 16 + lq * 4 + i) * TS + t * 16 + lr] = acc[rb][t][i];
      }
    } else {
      const float* p0 = d.partials + (int64_t)tile_id * d.splits * (NT * MT);
      switch (d.splits) {
        case 2: sum_partials<2, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        case 3: sum_partials<3, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        case 4: sum_partials<4, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        case 5: sum_partials<5, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        case 6: sum_partials<6, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        case 7: sum_partials<7, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
        default: sum_partials<8, NT * MT / 4, MT, TS, NTH, EH, DUAL, NB>(p0, tile, h); break;
      }
    }
    __syncthreads();
    if constexpr (SAMPLE)
      epi_sample(d, tile, TS, TCH, col0 + h * TCH, m0, mv, MT, s_scale);
    else
      run_epilogue<(TCH + 63) / 64, false, TOPK_TILE>(d, tile, TS, TCH, col0 + h * TCH, m0, mv, MT, s_scale, (float*)s_red,
                                           &s_flag, n_epi);
  }
}

// ---------------------------------------------------------------------------------
// fp32 VALU kernel (fp32 layers): tile of 64 weight rows x 32 tokens, whole K.
// ---------------------------------------------------------------------------------
// K goes through LDS in chunks of F32_KC: a chunk's W (64 x 64) and X (32 x 64) are read with
// 16-byte loads, and the next chunk's loads are issued before this chunk's math (register
// double buffering), so the chunk loop costs one memory round trip in total rather than one
// per chunk.  Thread (tr = tid % 16, tt = tid / 16) accumulates weight rows tr + 16 i (i < 4)
// for tokens tt and tt + 16 from 16-byte LDS reads along k: 6 reads feed 32 FMAs.
constexpr int F32_NT = 64, F32_MT = 32, F32_KC = 64;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d, int grid_real) {
  constexpr int TS = F32_MT + 4;
  constexpr int KP = F32_KC + 4;  // LDS row stride (floats): rows stay 16-byte aligned, reads conflict-free
  __shared__ __align__(16) float xs[F32_MT][KP];
  __shared__ __align__(16) float ws[F32_NT][KP];
  __shared__ float tile[F32_NT * TS];
  __shared__ float s_scale[F32_MT];
  __shared__ float s_ssq[F32_MT];
  __shared__ unsigned long long s_red[256];
  __shared__ int s_flag;
  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  if (bid >= grid_real) return;
  const int tid = threadIdx.x;
  const int m_tiles = (d.m + F32_MT - 1) / F32_MT;
  const int mt_i = bid % m_tiles, nt_i = bid / m_tiles;
  const int col0 = nt_i * F32_NT, m0 = mt_i * F32_MT;
  const int mv = min(F32_MT, d.m - m0);
  // staging: W piece u (< 4) of this thread = row tid / 16 + 16 u, columns 4 (tid % 16) .. + 3;
  // X = token tid / 8, columns 8 (tid % 8) .. + 7
  const int wg = tid % 16, wr0 = tid / 16;
  const float* wrow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rr = wr0 + 16 * u;
    const bool second = d.dual && rr >= F32_NT / 2;
    const int row = d.dual ? (col0 / 2 + (rr % (F32_NT / 2))) : col0 + rr;
    const int nrows = d.n;
    wrow[u] = row < nrows ? (const float*)(second ? d.w1 : d.w0) + (int64_t)row * d.ldw : nullptr;
  }
  const int xt = tid / 8, xg = tid % 8;
  const bool xlive = m0 + xt < d.m;
  float4 wv[4];
  float xv[8];
  float ssq = 0.f;
  auto load = [&](int kc) {
    const int kw = kc + 4 * wg;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      wv[u] = (wrow[u] && kw < d.k) ? *(const float4*)(wrow[u] + kw) : make_float4(0.f, 0.f, 0.f, 0.f);
    const int kx = kc + 8 * xg;
#pragma unroll
    for (int q = 0; q < 8; ++q) xv[q] = 0.f;
    if (xlive && kx < d.k) load_x8(d.x, m0 + xt, kx, xv);
  };
  auto store = [&](int kc) {
#pragma unroll
    for (int u = 0; u < 4; ++u) *(float4*)&ws[wr0 + 16 * u][4 * wg] = wv[u];
    const int kx = kc + 8 * xg;
#pragma unroll
    for (int q = 0; q < 8; ++q) ssq += xv[q] * xv[q];
    if (kx < d.k) apply_gain8(d.x, kx, xv);
    *(float4*)&xs[xt][8 * xg] = make_float4(xv[0], xv[1], xv[2], xv[3]);
    *(float4*)&xs[xt][8 * xg + 4] = make_float4(xv[4], xv[5], xv[6], xv[7]);
  };
  const int tr = tid % 16, tt = tid / 16;
  float acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = 0.f;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < d.k; kc += F32_KC) {
    const bool more = kc + F32_KC < d.k;
    if (more) load(kc + F32_KC);
#pragma unroll 4
    for (int kk = 0; kk < F32_KC; kk += 4) {
      float4 w4[4], x4[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = *(const float4*)&ws[tr + 16 * i][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) x4[j] = *(const float4*)&xs[tt + 16 * j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] += w4[i].x * x4[j].x + w4[i].y * x4[j].y + w4[i].z * x4[j].z + w4[i].w * x4[j].w;
    }
    __syncthreads();
    if (more) {
      store(kc + F32_KC);
      __syncthreads();
    }
  }
  // row sums of squares: the 8 staging threads of a token are adjacent lanes
  ssq += __shfl_xor(ssq, 1, 64);
  ssq += __shfl_xor(ssq, 2, 64);
  ssq += __shfl_xor(ssq, 4, 64);
  if (xg == 0) s_ssq[xt] = ssq;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) tile[(tr + 16 * i) * TS + tt + 16 * j] = acc[i][j];
  __syncthreads();
  if (tid < F32_MT) s_scale[tid] = d.x.norm ? rsqrtf(s_ssq[tid] / (float)d.k + d.x.eps) : 1.f;
  __syncthreads();
  const int tc = d.dual ? F32_NT / 2 : F32_NT;
  const int c0 = d.dual ? col0 / 2 : col0;
  run_epilogue<(F32_NT + 63) / 64, true, false>(d, tile, TS, tc, c0, m0, mv, F32_MT, s_scale, (float*)s_red, &s_flag,
                                         grid_real);
}

struct CfgInfo {
  int nw, rb, pd, mt, kc, eh;
};
// 0-2: 64-token tiles for a few dozen rows (weight streaming); 3, 4: 128- and 256-token
// tiles for hundreds of rows; 5, 6: 256 weight rows x 192 / 160 tokens with the epilogue in
// two halves (every weight byte read once for up to 256 rows, two 16-row blocks per wave).
// Config 5 has no gate/up instance (it would spill registers).  7, 8: wide tiles (four
// waves, 32x32x16 MFMAs, 256 weight rows x 192 / 160 tokens) for LM heads only, one K split.
// 9: 16-token tiles for up to 16 rows (decode steps, small draft levels): a quarter of the
// X staging and of the split-K partials of the 64-token tile.  10: 32-token tiles, taken
// from the measured table only (two token tiles per weight tile for 33..64 rows: twice the
// workgroups, the second read of each weight tile served by the XCD's L2).
constexpr int kNumCfgs = 11;
constexpr CfgInfo kCfgs[kNumCfgs] = {{8, 4, 4, 64, 512, 1},   {8, 2, 4, 64, 512, 1},   {8, 1, 8, 64, 512, 1},
                                     {8, 2, 4, 128, 256, 1},  {8, 1, 4, 256, 128, 1},  {8, 2, 4, 192, 128, 2},
                                     {8, 2, 4, 160, 128, 2},  {4, 4, 4, 192, 128, 2},  {4, 4, 4, 160, 128, 2},
                                     {8, 1, 8, 16, 512, 1},   {8, 1, 8, 32, 512, 1}};
constexpr bool cfg_wide(int c) { return c == 7 || c == 8; }

template <int NW, int RB, int PD, bool DUAL, int MT, int KC, int XB, int EH = 1>
void launch_cfg(const GemmDesc& d, int grid, hipStream_t s) {
  const int padded = (grid + kXcds - 1) / kXcds * kXcds;
  if constexpr (!DUAL) {
    if (d.epi.kind == EPI_SAMPLE) {
      hipLaunchKernelGGL((gemm_bf16_kernel<NW, RB, PD, false, MT, KC, XB, EH, true>), dim3(padded), dim3(NW * 64), 0,
                         s, d, grid);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<NW, RB, PD, DUAL, MT, KC, XB, EH, false>), dim3(padded), dim3(NW * 64), 0, s,
                     d, grid);
}

}  // namespace

GemmPlan plan_gemm(int dtype, int n, int k, int m, int dual, int epi_kind, int head_dim) {
  GemmPlan p{};
  if (dtype == EAGLE_F32) {
    p.cfg = 100;
    p.splits = 1;
    p.kps = k;
    p.tile_rows = F32_NT;
    p.tile_cols = dual ? F32_NT / 2 : F32_NT;
    p.mt = F32_MT;
    p.n_tiles = (n + p.tile_cols - 1) / p.tile_cols;
    p.w_tiles = p.n_tiles;
    p.m_tiles = (m + F32_MT - 1) / F32_MT;
    return p;
  }
  // Cost model (microseconds), fitted (least squares on log time) to the measured launch
  // times of every tile configuration and K split at the 8B- and 70B-shaped projections
  // with 16..960 tokens.  Workgroups run in rounds of 256 (each needs most of a CU's LDS).
  // Eight-wave tiles, per workgroup: its weight slice streams at min(45 GB/s, 7.4 TB/s /
  // resident workgroups) while its MFMAs run (2.4 TFLOP/s per CU with one 16-row block
  // per wave, 3.3 with more), plus a fixed ~4 us; split-K adds a serial tail: the last
  // workgroup of a tile reads every partial tile at ~40 GB/s, plus ~12 us.  Four-wave wide
  // tiles (one K split): 30 GB/s, 5.1 TFLOP/s per CU and ~40 us fixed, so they only pay
  // for themselves with hundreds of rows.  (The activation reads never limited the fit.)
  // The top-k epilogue costs ~0.75 us per 1000 (token, column) pairs of a tile.
  constexpr double kBcu = 44.7e3, kBchip = 7.38e6, kP1 = 2.36e6, kP2 = 3.33e6, kF0 = 3.9, kBfix = 39.5e3,
                   kFsplit = 12.2, kTopk = 7.5e-4;                   // bytes/us, flop/us, us
  constexpr double kBcuW = 29.9e3, kPW = 5.08e6, kF0W = 40.3;        // wide tiles
  double best = 1e30;
  int best_c = -1, best_s = 1;
  // (the 16-token tile is tried first, so it wins the ties: with one K split its cost is
  // the 64-token tile's, while it stages a quarter of the activations; measured 7% faster
  // for the 8B gate/up at 1..16 rows)
  static constexpr int kOrder[kNumCfgs] = {9, 0, 1, 2, 3, 4, 5, 6, 7, 8, 10};
  for (int ci = 0; ci < kNumCfgs; ++ci) {
    const int c = kOrder[ci];
    if (c == 10) continue;  // (measured picks only)
    const CfgInfo& cf = kCfgs[c];
    const bool wide = cfg_wide(c);
    if (wide && (m < 192 || epi_kind == EPI_TOPK)) continue;  // never faster below a few hundred rows
    // 16-token tiles: for at most 16 rows (decode, small draft levels); the top-k and
    // sampling epilogues split a tile's tokens over at most 8 thread groups (>= 64 tokens)
    if (cf.mt < 64 && (m > cf.mt || epi_kind == EPI_TOPK || epi_kind == EPI_SAMPLE)) continue;
    if (epi_kind == EPI_TOPK && cf.mt > 160) continue;  // the top-k epilogue is not compiled into these
    const int nt = cf.nw * cf.rb * 16;
    const int tc = dual ? nt / 2 : nt;
    if (epi_kind == EPI_QKV && (tc / cf.eh) % head_dim) continue;
    if (dual && c == 5) continue;  // no gate/up instance
    const int m_tiles = (m + cf.mt - 1) / cf.mt;
    const int kchunks = (k + cf.kc - 1) / cf.kc;
    const int tiles = ((n + tc - 1) / tc) * m_tiles;
    for (int s = 1; s <= (wide ? 1 : std::min(kchunks, 8)); ++s) {
      const int cps = (kchunks + s - 1) / s;  // chunks per split
      const int se = (kchunks + cps - 1) / cps;
      if (se != s) continue;
      const double kps = (double)cps * cf.kc;
      const int G = tiles * se;
      const int rounds = (G + 255) / 256;
      const double bw = std::min(wide ? kBcuW : kBcu, kBchip / std::min(G, 256));
      const double flops = 2.0 * nt * cf.mt * kps;
      const double part = (double)nt * cf.mt * 4;
      double per = std::max(nt * kps * 2 / bw, flops / (wide ? kPW : cf.rb == 1 ? kP1 : kP2)) + (wide ? kF0W : kF0);
      if (epi_kind == EPI_TOPK) per += kTopk * cf.mt * tc;
      double cost = rounds * per;
      if (se > 1) cost += se * part / kBfix + kFsplit;
      if (cost < best * 0.999) {
        best = cost;
        best_c = c;
        best_s = se;
      }
    }
  }
  // Shapes where the model's pick was measured well behind the best (tile configuration,
  // K split) of a sweep over all of them (the 8B- and 70B-shaped projections, rows 16..960),
  // confirmed by alternating runs of both picks: the measured best is taken for row counts
  // within 25% of the swept one.  In the 160..256-row range of the draft's levels: QKV at
  // 256 rows, O at 256 and down at 160 rows 6-20% faster than the model's 128-row tiles with
  // few K splits, the draft's feature FC 3-4%; the 8B QKV at 160 rows on 32-token tiles
  // (five token tiles per weight tile, one K split) 19% faster than the 64-token tiles the
  // table gave it before the weight stream took the non-temporal hint.  At 60 rows (one
  // verified tree) the 8B QKV, O and down on 32-token tiles: 8%, 16% and 7% faster (50-60
  // rows; at 75 rows, three token tiles, O and down were slower, so those picks stop at two
  // token tiles; the 70B shapes gained nothing).  The 8B gate/up at 160 rows now takes the
  // model's pick (3% faster than the 128-token tiles measured best without the hint).  For
  // hundreds of rows: the 8B O at 362 and 960 rows on 256-row x 64-token tiles (9% and 5%
  // faster) and the QKV at 960 rows on 512-row tiles (2%).
  struct TunedPick {
    int n, k, dual, epi, m, cfg, splits;
  };
  static constexpr TunedPick kTuned[] = {
      {6144, 4096, 0, EPI_QKV, 160, 10, 1},   {6144, 4096, 0, EPI_QKV, 256, 1, 2},
      {4096, 4096, 0, EPI_RESID, 256, 2, 2},  {4096, 14336, 0, EPI_RESID, 160, 1, 5},
      {10240, 8192, 0, EPI_QKV, 160, 1, 2},   {8192, 8192, 0, EPI_RESID, 160, 3, 4},
      {4096, 8192, 0, EPI_RESID, 160, 1, 4},
      {6144, 4096, 0, EPI_QKV, 60, 10, 2},    {4096, 4096, 0, EPI_RESID, 60, 10, 4},
      {4096, 14336, 0, EPI_RESID, 60, 10, 4},
      {4096, 4096, 0, EPI_RESID, 362, 1, 2},  {4096, 4096, 0, EPI_RESID, 960, 1, 1},
      {6144, 4096, 0, EPI_QKV, 960, 0, 1}};
  {
    double bestd = 0.2232;  // |ln(m / swept m)| <= ln 1.25
    for (const TunedPick& t : kTuned) {
      if (t.n != n || t.k != k || t.dual != dual || t.epi != epi_kind) continue;
      // a narrow-tile pick measured with at most two token tiles does not extend to more
      if (kCfgs[t.cfg].mt < 64 && t.m <= 2 * kCfgs[t.cfg].mt && m > 2 * kCfgs[t.cfg].mt) continue;
      const double dd = std::fabs(std::log((double)m / t.m));
      if (dd <= bestd) {
        bestd = dd;
        best_c = t.cfg;
        best_s = t.splits;
      }
    }
  }
  // LM heads of 320+ rows (argmax or sampling epilogue): the wide tiles were measured
  // 1.5-2% faster than the best eight-wave tile from 360 to 960 rows; of the two token
  // tiles, the one that pads fewer rows (ties: the wider one).
  if (!dual && n >= 32768 && m >= 320 && (epi_kind == EPI_ARGMAX || epi_kind == EPI_SAMPLE)) {
    const int pad7 = (m + kCfgs[7].mt - 1) / kCfgs[7].mt * kCfgs[7].mt;
    const int pad8 = (m + kCfgs[8].mt - 1) / kCfgs[8].mt * kCfgs[8].mt;
    best_c = pad8 < pad7 ? 8 : 7;
    best_s = 1;
  }
  if (best_c < 0) {  // no tile shape fits (the launch then refuses the plan)
    p.cfg = -1;
    return p;
  }
  const CfgInfo& cf = kCfgs[best_c];
  const int kchunks = (k + cf.kc - 1) / cf.kc;
  p.cfg = best_c;
  p.splits = best_s;
  p.kps = ((kchunks + best_s - 1) / best_s) * cf.kc;
  p.tile_rows = cf.nw * cf.rb * 16;
  const int wcols = dual ? p.tile_rows / 2 : p.tile_rows;  // output columns per weight tile
  p.tile_cols = wcols / cf.eh;
  p.mt = cf.mt;
  p.w_tiles = (n + wcols - 1) / wcols;
  p.n_tiles = p.w_tiles * cf.eh;
  p.m_tiles = (m + cf.mt - 1) / cf.mt;
  return p;
}

void gemm_workspace(const GemmPlan& p, size_t* partial_floats, size_t* sumsq_floats, size_t* counter_ints) {
  const size_t tiles = (size_t)p.w_tiles * p.m_tiles;
  if (p.splits > 1) {
    *partial_floats = tiles * p.splits * p.tile_rows * p.mt;
    *sumsq_floats = tiles * p.splits * p.mt;
    *counter_ints = tiles;
  } else {
    *partial_floats = 0;
    *sumsq_floats = 0;
    *counter_ints = 0;
  }
}

int launch_gemm(GemmDesc& d, const GemmPlan& p, hipStream_t s) {
  d.cfg = p.cfg;
  d.splits = p.splits;
  d.kps = p.kps;
  if (d.k % 32 || (d.x.ka % 8) || p.cfg < 0 || (p.cfg != 100 && p.cfg >= kNumCfgs)) return EAGLE_ERR_UNSUPPORTED;
  if (p.cfg != 100 && (d.x.a.dtype != EAGLE_BF16 || d.x.b.dtype != EAGLE_BF16)) return EAGLE_ERR_UNSUPPORTED;
  if (p.cfg == 100 && d.epi.kind == EPI_TOPK) return EAGLE_ERR_UNSUPPORTED;  // its LDS tile is too small
  if (d.epi.kind == EPI_TOPK && d.n > (1 << 20)) return EAGLE_ERR_UNSUPPORTED;  // 20-bit columns in the keys
  if (p.cfg != 100) {
    // top-k: compiled into the eight-wave tiles of 64..160 tokens; sampling: >= 64 tokens
    const int mt = kCfgs[p.cfg].mt;
    if (d.epi.kind == EPI_TOPK && (cfg_wide(p.cfg) || mt > 160 || mt < 64)) return EAGLE_ERR_UNSUPPORTED;
    if (d.epi.kind == EPI_SAMPLE && mt < 64) return EAGLE_ERR_UNSUPPORTED;
  }
  if (p.cfg == 100 && d.w_layout) return EAGLE_ERR_UNSUPPORTED;              // fragment blocks are bf16
  if (d.dual && d.epi.kind == EPI_SAMPLE) return EAGLE_ERR_UNSUPPORTED;
  const int grid = p.w_tiles * p.m_tiles * p.splits;
  if (grid <= 0) return EAGLE_OK;
  if (p.cfg == 100) {
    const int padded = (grid + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(padded), dim3(256), 0, s, d, grid);
  } else {
    const bool dual = d.dual != 0;
    switch (p.cfg) {
      case 0: dual ? launch_cfg<8, 4, 4, true, 64, 512, 2>(d, grid, s) : launch_cfg<8, 4, 4, false, 64, 512, 2>(d, grid, s); break;
      case 1: dual ? launch_cfg<8, 2, 4, true, 64, 512, 2>(d, grid, s) : launch_cfg<8, 2, 4, false, 64, 512, 2>(d, grid, s); break;
      case 2: dual ? launch_cfg<8, 1, 8, true, 64, 512, 2>(d, grid, s) : launch_cfg<8, 1, 8, false, 64, 512, 2>(d, grid, s); break;
      case 3: dual ? launch_cfg<8, 2, 4, true, 128, 256, 2>(d, grid, s) : launch_cfg<8, 2, 4, false, 128, 256, 2>(d, grid, s); break;
      case 4: dual ? launch_cfg<8, 1, 4, true, 256, 128, 2>(d, grid, s) : launch_cfg<8, 1, 4, false, 256, 128, 2>(d, grid, s); break;
      case 5:
        if (dual) return EAGLE_ERR_UNSUPPORTED;
        launch_cfg<8, 2, 4, false, 192, 128, 2, 2>(d, grid, s);
        break;
      case 6: dual ? launch_cfg<8, 2, 4, true, 160, 128, 2, 2>(d, grid, s) : launch_cfg<8, 2, 4, false, 160, 128, 2, 2>(d, grid, s); break;
      case 7:
      case 8:
        // wide tiles: a single K split only
        if (p.splits != 1) return EAGLE_ERR_UNSUPPORTED;
        if (p.cfg == 7)
          dual ? launch_cfg<4, 4, 4, true, 192, 128, 2, 2>(d, grid, s) : launch_cfg<4, 4, 4, false, 192, 128, 2, 2>(d, grid, s);
        else
          dual ? launch_cfg<4, 4, 4, true, 160, 128, 2, 2>(d, grid, s) : launch_cfg<4, 4, 4, false, 160, 128, 2, 2>(d, grid, s);
        break;
      case 9: dual ? launch_cfg<8, 1, 8, true, 16, 512, 2>(d, grid, s) : launch_cfg<8, 1, 8, false, 16, 512, 2>(d, grid, s); break;
      case 10: dual ? launch_cfg<8, 1, 8, true, 32, 512, 2>(d, grid, s) : launch_cfg<8, 1, 8, false, 32, 512, 2>(d, grid, s); break;
      default: return EAGLE_ERR_UNSUPPORTED;
    }
  }
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

namespace {
// One 16-byte fragment piece per thread: piece f = (step s, block b, lane l) in that order.
__global__ __launch_bounds__(256) void pack_fragments_kernel(const bf16* __restrict__ w, int rows, int cols,
                                                              bf16* __restrict__ out, int64_t pieces) {
  const int nblk = (rows + 15) / 16;
  for (int64_t f = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; f < pieces; f += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(f % 64);
    const int64_t sb = f / 64;
    const int b = (int)(sb % nblk);
    const int s = (int)(sb / nblk);
    const int row = b * 16 + l % 16, col = s * 32 + (l / 16) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < rows) v = *(const uint4*)(w + (int64_t)row * cols + col);
    *(uint4*)(out + f * 8) = v;
  }
}
}  // namespace

void launch_pack_fragments(const void* w, int rows, int cols, void* out, hipStream_t s) {
  const int64_t pieces = (int64_t)((rows + 15) / 16) * (cols / 32) * 64;
  const int grid = (int)std::min<int64_t>((pieces + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_fragments_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)w, rows, cols, (bf16*)out,
                     pieces);
}

}  // namespace eagle
