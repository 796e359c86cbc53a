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

// Rotary angle pos * theta^(-2j/hd): argument built in fp64 and reduced to [-pi, pi]
// before the fp32 sincos, so positions up to 10^5 keep full fp32 accuracy.
__device__ __forceinline__ void rope_cs(int pos, int j, int hd, float theta, float* c, float* s) {
  const double inv = exp2(-(2.0 * j / hd) * log2((double)theta));
  const double a = (double)pos * inv;
  const double twopi = 6.283185307179586476925286766559;
  const double r = a - rint(a / twopi) * twopi;
  sincosf((float)r, s, c);
}

// Fused epilogue over a finished fp32 tile in LDS: tile[r * ts + t] is output column
// col0 + r (for dual tiles: gate columns r < tc, up columns r >= tc) of token m0 + t,
// before the per-row norm scale scale[t].
__device__ void run_epilogue(const GemmDesc& d, const float* tile, int ts, int tc, int col0, int m0, int mv,
                             int mt, const float* scale, float* red_scratch, int* s_flag, int n_epi) {
  const Epi& e = d.epi;
  const int tid = threadIdx.x, nth = blockDim.x;
  switch (e.kind) {
    case EPI_STORE_F32:
    case EPI_RESID: {
      for (int i = tid; i < tc * mv; i += nth) {
        const int r = i % tc, t = i / tc;
        const int c = col0 + r;
        if (c >= d.n) continue;
        float v = scale[t] * tile[r * ts + t];
        if (e.kind == EPI_RESID) {
          const int64_t rrow = e.resid_idx ? (int64_t)e.resid_idx[m0 + t] : (int64_t)(m0 + t);
          v += load_elem(e.resid, e.resid_dtype, rrow * e.ld_resid + c);
        }
        e.out[(int64_t)(m0 + t) * e.ld_out + c] = v;
      }
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
      const int hd = e.hd, half = hd / 2;
      const int heads_in_tile = tc / hd;
      for (int i = tid; i < mv * heads_in_tile * half; i += nth) {
        const int j = i % half;
        const int hl = (i / half) % heads_in_tile;
        const int t = i / (half * heads_in_tile);
        const int head = col0 / hd + hl;
        if (head >= e.hq + 2 * e.hkv) continue;
        const int m = m0 + t;
        float a = scale[t] * tile[(hl * hd + j) * ts + t];
        float b = scale[t] * tile[(hl * hd + j + half) * ts + t];
        if (head < e.hq + e.hkv && e.theta > 0.f) {
          float c, s;
          rope_cs(e.pos[m], j, hd, e.theta, &c, &s);
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
          dst = e.k_out;
          base = ((int64_t)m * e.hkv + (head - e.hq)) * hd;
        } else {
          dst = e.v_out;
          base = ((int64_t)m * e.hkv + (head - e.hq - e.hkv)) * hd;
        }
        store_out(dst, e.out_dtype, base + j, a);
        store_out(dst, e.out_dtype, base + j + half, b);
      }
      break;
    }
    case EPI_ARGMAX: {
      // thread -> (token t, row stripe); rows are scanned in increasing order so the
      // first maximum wins, then stripes are merged through LDS with the packed key.
      const int stripes = nth / mt;
      const int t = tid % mt, st = tid / mt;
      unsigned long long best = 0ull;
      if (t < mv) {
        const float sc = scale[t];
        for (int r = st; r < tc; r += stripes) {
          const int c = col0 + r;
          if (c >= d.n) break;
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
      // the last workgroup of the launch unpacks the keys and clears them
      __syncthreads();
      if (tid == 0) {
        __threadfence();
        const int old = atomicAdd(e.done, 1);
        *s_flag = (old == n_epi - 1);
      }
      __syncthreads();
      if (*s_flag) {
        __threadfence();
        for (int m = tid; m < d.m; m += nth) {
          const unsigned long long key = __hip_atomic_load(&e.keys[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          e.argmax_out[m] = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
          if (e.max_out) e.max_out[m] = ord2f((uint32_t)(key >> 32));
          __hip_atomic_store(&e.keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) __hip_atomic_store(e.done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
    case EPI_TOPK: {
      // per token: this tile's top-k (value desc, index asc) and (max, sum exp(v - max))
      const int K = e.topk;
      const int n_tiles = (d.n + tc - 1) / tc;
      const int tile_i = col0 / tc;
      const int nw = nth / 64, w = tid / 64, lane = tid % 64;
      for (int t = w; t < mv; t += nw) {
        const float sc = scale[t];
        // (max, sumexp) over valid columns
        float mx = -INFINITY;
        for (int r = lane; r < tc && col0 + r < d.n; r += 64) mx = fmaxf(mx, sc * tile[r * ts + t]);
        mx = wave_max(mx);
        float se = 0.f;
        for (int r = lane; r < tc && col0 + r < d.n; r += 64) se += __expf(sc * tile[r * ts + t] - mx);
        se = wave_sum(se);
        const int64_t ob = ((int64_t)(m0 + t) * n_tiles + tile_i);
        if (lane == 0) {
          e.lse_part[ob * 2] = mx;
          e.lse_part[ob * 2 + 1] = se;
        }
        // top-k by repeated wave argmax, excluding the keys already chosen
        unsigned long long last = ~0ull;
        for (int q = 0; q < K; ++q) {
          unsigned long long bk = 0ull;
          for (int r = lane; r < tc && col0 + r < d.n; r += 64) {
            const unsigned long long key = argmax_key(sc * tile[r * ts + t], (uint32_t)(col0 + r));
            if (key < last && key > bk) bk = key;
          }
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long ok = __shfl_xor(bk, o, 64);
            bk = ok > bk ? ok : bk;
          }
          last = bk;
          if (lane == 0) {
            const bool valid = bk != 0ull;
            e.topk_val[ob * K + q] = valid ? ord2f((uint32_t)(bk >> 32)) : -INFINITY;
            e.topk_idx[ob * K + q] = valid ? (int32_t)(0xffffffffu - (uint32_t)(bk & 0xffffffffull)) : -1;
          }
        }
      }
      break;
    }
    default:
      break;
  }
}

// ---------------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------------
template <int NW, int RB, int PD, int MT, int KC, bool DUAL>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(GemmDesc d, int grid_real) {
  constexpr int NT = NW * RB * 16;        // weight rows per tile (both blocks when DUAL)
  constexpr int TC = DUAL ? NT / 2 : NT;  // output columns per tile
  constexpr int NSTEP = KC / 32;
  constexpr int XS = KC + 8;              // LDS row stride of the X chunk (bf16)
  constexpr int TS = MT + 4;              // LDS row stride of the output tile (f32)
  constexpr int LDS_X = MT * XS * 2;
  constexpr int LDS_T = NT * TS * 4;
  constexpr int LDS = LDS_X > LDS_T ? LDS_X : LDS_T;
  constexpr int RPW = MT / NW;            // X rows staged per wave
  constexpr int NTH = NW * 64;
  static_assert(NSTEP % PD == 0, "prefetch depth must divide the chunk steps");
  static_assert(MT % NW == 0 && MT % 16 == 0, "token tile");

  __shared__ __align__(16) unsigned char smem[LDS];
  __shared__ float s_scale[MT];
  __shared__ float s_ssq[MT];
  __shared__ unsigned long long s_red[NTH];
  __shared__ int s_flag;

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  if (bid >= grid_real) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;

  const int m_tiles = (d.m + MT - 1) / MT;
  int b = bid;
  const int split = b % d.splits;
  b /= d.splits;
  const int mt_i = b % m_tiles;
  const int nt_i = b / m_tiles;
  const int col0 = nt_i * TC, m0 = mt_i * MT;
  const int mv = min(MT, d.m - m0);
  const int kps = (((d.k + d.splits - 1) / d.splits) + 31) & ~31;
  const int kb = split * kps;
  const int ke = min(d.k, kb + kps);

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
  const bf16* wp[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = min(wrow0 + rb * 16 + lr, d.n - 1);
    wp[rb] = wblk + (int64_t)row * d.ldw + lq * 8;
  }

  f32x4 acc[RB][MT / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < MT / 16; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weight prefetch ring.  Loads are unconditional (addresses past the K range are
  // clamped to its last step): a conditional load would make the compiler wait for it
  // before merging the ring register, which serialises the stream.
  const int klast = ke - 32;
  bf16x8_t wbuf[PD][RB];
#pragma unroll
  for (int s = 0; s < PD; ++s) {
    const int k = min(kb + s * 32, klast);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) wbuf[s][rb] = *(const bf16x8_t*)(wp[rb] + k);
  }

  float ssq[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) ssq[j] = 0.f;

  bf16* xl = (bf16*)smem;
  for (int kc = kb; kc < ke; kc += KC) {
    __syncthreads();
    // stage X[m0 .. m0+MT)[kc .. kc+KC) into LDS as bf16
    const int klen = min(KC, ke - kc);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = wid + j * NW;
      const int m = m0 + r;
      for (int g = lane; g < KC / 8; g += 64) {
        const int k = kc + g * 8;
        uint4 pk = make_uint4(0u, 0u, 0u, 0u);
        if (m < d.m && g * 8 < klen) {
          float v[8];
          load_x8(d.x, m, k, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) ssq[j] += v[i] * v[i];
          apply_gain8(d.x, k, v);
          pk = make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]), pack2bf(v[6], v[7]));
        }
        *(uint4*)(xl + r * XS + g * 8) = pk;
      }
    }
    __syncthreads();
    // Every chunk runs all NSTEP steps: past the K range X is zero in LDS, so the
    // extra steps of a short last chunk add exact zeros (and stay branch-free).
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      bf16x8_t cur[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) cur[rb] = wbuf[s % PD][rb];
      const int kn = min(kc + (s + PD) * 32, klast);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wbuf[s % PD][rb] = *(const bf16x8_t*)(wp[rb] + kn);
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

  // row sums of squares of this K range
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const float v = wave_sum(ssq[j]);
    if (lane == 0) s_ssq[wid + j * NW] = v;
  }
  __syncthreads();

  float* tile = (float*)smem;
  const int tile_id = nt_i * m_tiles + mt_i;
  if (d.splits == 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int t = 0; t < MT / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[((wid * RB + rb) * 16 + lq * 4 + i) * TS + t * 16 + lr] = acc[rb][t][i];
    if (tid < MT) s_scale[tid] = d.x.norm ? rsqrtf(s_ssq[tid] / (float)d.k + d.x.eps) : 1.f;
  } else {
    float* part = d.partials + ((int64_t)tile_id * d.splits + split) * (NT * MT);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int t = 0; t < MT / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[((wid * RB + rb) * 16 + lq * 4 + i) * MT + t * 16 + lr] = acc[rb][t][i];
    if (tid < MT) d.sumsq_part[((int64_t)tile_id * d.splits + split) * MT + tid] = s_ssq[tid];
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const int old = atomicAdd(&d.counters[tile_id], 1);
      s_flag = (old == d.splits - 1);
    }
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    const float* p0 = d.partials + (int64_t)tile_id * d.splits * (NT * MT);
    for (int i = tid; i < NT * MT; i += NTH) {
      float v = 0.f;
      for (int s = 0; s < d.splits; ++s) v += p0[(int64_t)s * NT * MT + i];
      tile[(i / MT) * TS + (i % MT)] = v;
    }
    if (tid < MT) {
      float v = 0.f;
      for (int s = 0; s < d.splits; ++s) v += d.sumsq_part[((int64_t)tile_id * d.splits + s) * MT + tid];
      s_scale[tid] = d.x.norm ? rsqrtf(v / (float)d.k + d.x.eps) : 1.f;
    }
    if (tid == 0) d.counters[tile_id] = 0;
  }
  __syncthreads();
  run_epilogue(d, tile, TS, TC, col0, m0, mv, MT, s_scale, (float*)s_red, &s_flag,
               ((d.n + TC - 1) / TC) * m_tiles);
}

// ---------------------------------------------------------------------------------
// fp32 VALU kernel (fp32 layers): tile of 64 weight rows x 32 tokens, whole K.
// ---------------------------------------------------------------------------------
constexpr int F32_NT = 64, F32_MT = 32, F32_KC = 64;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d, int grid_real) {
  constexpr int TS = F32_MT + 4;
  __shared__ float xs[F32_MT][F32_KC + 1];
  __shared__ float ws[F32_NT][F32_KC + 1];
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
  // thread computes rows r = tid % 64 and tokens t = tid / 64 + 4 * i
  const int r = tid % F32_NT, t0 = tid / F32_NT;
  float acc[F32_MT / 4];
  for (int i = 0; i < F32_MT / 4; ++i) acc[i] = 0.f;
  if (tid < F32_MT) s_ssq[tid] = 0.f;
  for (int kc = 0; kc < d.k; kc += F32_KC) {
    __syncthreads();
    for (int i = tid; i < F32_MT * (F32_KC / 8); i += 256) {
      const int rr = i / (F32_KC / 8), g = i % (F32_KC / 8);
      const int m = m0 + rr, k = kc + g * 8;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (m < d.m && k < d.k) {
        load_x8(d.x, m, k, v);
        float sq = 0.f;
        for (int q = 0; q < 8; ++q) sq += v[q] * v[q];
        atomicAdd(&s_ssq[rr], sq);
        apply_gain8(d.x, k, v);
      }
      for (int q = 0; q < 8; ++q) xs[rr][g * 8 + q] = v[q];
    }
    for (int i = tid; i < F32_NT * F32_KC; i += 256) {
      const int rr = i / F32_KC, kk = i % F32_KC;
      const int c = col0 + rr;
      const bool second = d.dual && rr >= F32_NT / 2;
      const int row = d.dual ? (col0 / 2 + (rr % (F32_NT / 2))) : c;
      const float* wsrc = (const float*)(second ? d.w1 : d.w0);
      const int nrows = d.n;
      ws[rr][kk] = (row < nrows && kc + kk < d.k) ? wsrc[(int64_t)row * d.ldw + kc + kk] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < F32_KC; ++kk) {
      const float wv = ws[r][kk];
      for (int i = 0; i < F32_MT / 4; ++i) acc[i] += wv * xs[t0 + 4 * i][kk];
    }
  }
  for (int i = 0; i < F32_MT / 4; ++i) tile[r * TS + t0 + 4 * i] = acc[i];
  __syncthreads();
  if (tid < F32_MT) s_scale[tid] = d.x.norm ? rsqrtf(s_ssq[tid] / (float)d.k + d.x.eps) : 1.f;
  __syncthreads();
  const int tc = d.dual ? F32_NT / 2 : F32_NT;
  const int c0 = d.dual ? col0 / 2 : col0;
  run_epilogue(d, tile, TS, tc, c0, m0, mv, F32_MT, s_scale, (float*)s_red, &s_flag, grid_real);
}

struct CfgInfo {
  int nw, rb, mt;
};
constexpr CfgInfo kCfgs[4] = {{8, 4, 64}, {8, 2, 64}, {8, 1, 64}, {4, 1, 64}};

template <int NW, int RB, int PD, bool DUAL>
void launch_cfg(const GemmDesc& d, int grid, hipStream_t s) {
  const int padded = (grid + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_bf16_kernel<NW, RB, PD, 64, 512, DUAL>), dim3(padded), dim3(NW * 64), 0, s, d, grid);
}

}  // namespace

GemmPlan plan_gemm(int dtype, int n, int k, int m, int dual, int epi_kind, int head_dim) {
  GemmPlan p{};
  if (dtype == EAGLE_F32) {
    p.cfg = 100;
    p.splits = 1;
    p.tile_rows = F32_NT;
    p.tile_cols = dual ? F32_NT / 2 : F32_NT;
    p.mt = F32_MT;
    p.n_tiles = (n + p.tile_cols - 1) / p.tile_cols;
    p.m_tiles = (m + F32_MT - 1) / F32_MT;
    return p;
  }
  const int mt = 64;
  const int m_tiles = (m + mt - 1) / mt;
  int chosen = -1;
  for (int c = 0; c < 4; ++c) {
    const int nt = kCfgs[c].nw * kCfgs[c].rb * 16;
    const int tc = dual ? nt / 2 : nt;
    if (epi_kind == EPI_QKV && tc % head_dim) continue;
    const int tiles = ((n + tc - 1) / tc) * m_tiles;
    if (tiles >= 240) {
      chosen = c;
      break;
    }
  }
  int splits = 1;
  if (chosen < 0) {
    chosen = 2;
    const int nt = kCfgs[chosen].nw * kCfgs[chosen].rb * 16;
    const int tc = dual ? nt / 2 : nt;
    const int tiles = ((n + tc - 1) / tc) * m_tiles;
    splits = (256 + tiles - 1) / tiles;
    splits = std::max(1, std::min(splits, k / 512));
  }
  p.cfg = chosen;
  p.splits = splits;
  p.tile_rows = kCfgs[chosen].nw * kCfgs[chosen].rb * 16;
  p.tile_cols = dual ? p.tile_rows / 2 : p.tile_rows;
  p.mt = mt;
  p.n_tiles = (n + p.tile_cols - 1) / p.tile_cols;
  p.m_tiles = m_tiles;
  // splits must each cover >= 32 k
  const int kps = (((k + p.splits - 1) / p.splits) + 31) & ~31;
  p.splits = (k + kps - 1) / kps;
  return p;
}

void gemm_workspace(const GemmPlan& p, size_t* partial_floats, size_t* sumsq_floats, size_t* counter_ints) {
  const size_t tiles = (size_t)p.n_tiles * p.m_tiles;
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
  if (d.k % 32 || (d.x.ka % 8)) return EAGLE_ERR_UNSUPPORTED;
  const int grid = p.n_tiles * p.m_tiles * p.splits;
  if (grid <= 0) return EAGLE_OK;
  if (p.cfg == 100) {
    const int padded = (grid + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(padded), dim3(256), 0, s, d, grid);
  } else {
    const bool dual = d.dual != 0;
    switch (p.cfg) {
      case 0: dual ? launch_cfg<8, 4, 4, true>(d, grid, s) : launch_cfg<8, 4, 4, false>(d, grid, s); break;
      case 1: dual ? launch_cfg<8, 2, 4, true>(d, grid, s) : launch_cfg<8, 2, 4, false>(d, grid, s); break;
      case 2: dual ? launch_cfg<8, 1, 8, true>(d, grid, s) : launch_cfg<8, 1, 8, false>(d, grid, s); break;
      case 3: dual ? launch_cfg<4, 1, 8, true>(d, grid, s) : launch_cfg<4, 1, 8, false>(d, grid, s); break;
      default: return EAGLE_ERR_UNSUPPORTED;
    }
  }
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle
