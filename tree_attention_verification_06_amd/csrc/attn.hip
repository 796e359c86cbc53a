// Tree-masked GQA attention over [KV prefix ; tree nodes] (gfx950).
//
// Every drafted node attends to the whole committed prefix of its sequence and to
// the tree nodes on its own root path (ancestor bitmask, self included), so all nodes
// of a tree are verified in one pass.
//
// bf16 path (head_dim 128): for one (sequence, KV head) the query rows are the g query
// heads of every node (row = node * g + head-in-group), so a K/V tile is loaded once
// and used by all of them (GQA).  Split-KV: workgroup (b, kv head, chunk, row group)
// handles up to 128 query rows against one chunk of prefix keys, or against the tree
// keys (the last chunk), and writes fp32 partials (running max, sum, unnormalised o);
// a merge kernel combines the chunks in fixed order (deterministic).
//  * K and V tiles (64 keys) are read with 16-byte coalesced loads two tiles ahead
//    (a register ring) and stored to double-buffered LDS in their natural [key][d]
//    layout with 16-byte writes: one barrier per tile.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 d from LDS, B = Q held
//    in registers); each lane then owns 4 consecutive keys of one query row, so the
//    row max needs only two cross-lane swaps and the softmax rescale of the output is
//    lane-local.
//  * O^T += V^T P^T with the same MFMA: B = P packed to bf16 in registers (exactly the
//    lane layout the score MFMA produced: k-slots 8q..8q+7 of lane group q are keys
//    4q..4q+3 and 16+4q..16+4q+3 of a 32-key step), A = V^T read from the natural V tile
//    with the gfx950 LDS transpose read (ds_read_b64_tr_b16): within a 16-lane group,
//    output lane 4a+c receives element c of the 8-byte pieces addressed by lanes a, a+4,
//    a+8, a+12, so lane s of group q addresses key 4q + s/4, d 4(s%4) of the d-block.
//  * tree keys are masked with the node's ancestor words: key j is visible iff bit j.
// fp32 path: a plain VALU kernel, one wave per (node, query head).
#include "attn.h"

#include <algorithm>
#include <type_traits>

namespace eagle {

namespace {

constexpr int kXcds = 8;
constexpr int RBW = 1;                  // 16-row query blocks per wave
constexpr int KT = 64;                  // keys per LDS tile
constexpr int HD = 128;
constexpr int KS = HD + 16;             // LDS row stride of the K tile (bf16): 288 bytes, an
                                        // odd multiple of 32, keeps the score reads (16 rows x
                                        // four 16-byte groups) free of bank conflicts
constexpr int VS = HD + 16;             // LDS row stride of the V tile (bf16): the four keys
                                        // of one transpose read land in distinct banks
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one gfx950 v_cvt_pk_bf16_f32; a in the
// low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that hold one query row)
// with the gfx950 lane swaps, which stay in the VALU (a shuffle would be an LDS round trip).
__device__ __forceinline__ float max_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ int remap_xcd(int b, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  return (b % kXcds) * per + b / kXcds;
}

// NWA waves per workgroup (NWA * 16 query rows): 8, or 4 for (b, kv head) pairs with few
// query rows, where two workgroups then share a CU (LDS and registers allow it) and one
// streams while the other waits.  PAGED: the cache is a page pool addressed through
// a.table (see CacheView); the contiguous instantiation is unchanged code.
template <int NWA, bool PAGED>
__global__ __launch_bounds__(NWA * 64, 2) void tree_attn_bf16_kernel(AttnArgs a, int grid_real) {
  constexpr int ROWS_WG = NWA * RBW * 16;  // query rows per workgroup
  __shared__ __align__(16) bf16 ks[2][KT * KS];
  __shared__ __align__(16) bf16 vs[2][KT * VS];

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  if (bid >= grid_real) return;
  int t = bid;
  const int rg = t % a.row_groups;
  t /= a.row_groups;
  const int c = t % a.n_chunks;
  t /= a.n_chunks;
  const int kvh = t % a.hkv;
  const int b = t / a.hkv;

  const int off = a.tree_off[b];
  const int N = a.n_nodes ? a.n_nodes[b] : a.tree_off[b + 1] - off;
  const int qlo = a.q_lo ? a.q_lo[b] : 0;
  const int g = a.hq / a.hkv;
  const int R = (N - qlo) * g;
  const int row_base = rg * ROWS_WG;
  if (row_base >= R || N - qlo > a.max_nodes || N > 64 * a.mw) return;
  const int P = min(max(a.prefix_len[b], 0), a.cap);
  const bool tree_chunk = (c == a.n_chunks - 1);
  int k0, k1;
  if (tree_chunk) {
    k0 = 0;
    k1 = N;
  } else {
    // the last prefix chunk takes every key up to P: the grid is planned for the host's
    // max_prefix, and a longer device prefix is then still attended in full
    k0 = c * a.kch;
    k1 = (c == a.n_chunks - 2) ? P : min(P, k0 + a.kch);
    if (k0 >= k1) return;
  }

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const bf16* q = (const bf16*)a.q;

  // Visibility words per query row: the tree chunk uses the node's ancestor words
  // (key j visible iff bit j); prefix chunks see every key, so their words are all ones.
  // Keeping the mask arithmetic free of branches matters: a branch between a score
  // MFMA and the read of its accumulator has been seen to lose the required wait states.
  bf16x8_t qf[RBW][4];
  uint64_t vis0[RBW], vis1[RBW];
#pragma unroll
  // Loads are unconditional (rows past R read row R - 1, which exists since row_base < R,
  // and are then given a zero query and an all-visible mask): a load under a branch would
  // be waited for at the join, before the first K/V loads could be issued.
  for (int j = 0; j < RBW; ++j) {
    const int row = row_base + (w * RBW + j) * 16 + lr;
    const bool live = row < R;
    const int rc = live ? row : R - 1;
    const int node = qlo + rc / g, hh = rc % g;
    const int64_t qrow = a.q_stride ? (int64_t)b * a.q_stride + (node - qlo) : (int64_t)(off + node);
    const bf16* qp = q + (qrow * a.hq + kvh * g + hh) * HD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8_t v = *(const bf16x8_t*)(qp + kk * 32 + lq * 8);
      qf[j][kk] = live ? v : bf16x8_t{};
    }
    const uint64_t* ap = a.anc + (int64_t)(off + node) * a.mw;
    const uint64_t a0 = ap[0];
    const uint64_t a1 = ap[a.mw > 1 ? 1 : 0];
    vis0[j] = (tree_chunk && live) ? a0 : ~0ull;
    vis1[j] = (tree_chunk && live) ? (a.mw > 1 ? a1 : 0ull) : ~0ull;
  }

  f32x4 o[RBW][8];
  float mrow[RBW], lsum[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    mrow[j] = -INFINITY;
    lsum[j] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // scores in log2 units: q.k / sqrt(128) * log2(e)
  const float sl2 = 0.08838834764831845f * 1.4426950408889634f;

  // contiguous: the (b, kv head) row base; paged: the kv head's offset within a page
  const int64_t cbase = (PAGED ? 0 : (int64_t)b * a.cb) + (int64_t)kvh * a.ch;
  const bf16* kc = (const bf16*)a.k_cache + cbase;
  const bf16* vc = (const bf16*)a.v_cache + cbase;
  const bf16* kt_base = (const bf16*)a.k_tree + ((int64_t)off * a.hkv + kvh) * HD;
  const bf16* vt_base = (const bf16*)a.v_tree + ((int64_t)off * a.hkv + kvh) * HD;
  const int64_t tree_stride = (int64_t)a.hkv * HD;

  // K/V tiles go global -> registers -> LDS.  The loads of tile i + 2 are issued before
  // the math of tile i, into the register slot whose tile was stored to LDS one step
  // earlier, so two tiles of math cover each load's latency.  Loads are unconditional
  // (keys past the chunk are clamped to its last key and zeroed when stored).
  constexpr int GPT = KT * 16 / (NWA * 64);  // 16-byte groups per thread per tensor
  uint4 kreg[2][GPT], vreg[2][GPT];
  // Addressing: thread row rowk = i >> 4 (a key within the tile) and 16-byte group gd = i & 15
  // are fixed per thread; a call's keys are kt0 + min(rowk, k1 - 1 - kt0) (clamped to the
  // chunk's last key), so the offset is a uniform base plus row * stride.  Paged: kt0 is a
  // multiple of 64 or the chunk's last key, and page sizes are multiples of 64, so every key
  // of a call lies in kt0's page: one (uniform) table lookup.  Tree chunks never consult the
  // table (their keys are node indices).
  const int64_t kst = tree_chunk ? tree_stride : a.ct;  // elements between consecutive keys
  const bf16* kb = (tree_chunk ? kt_base : kc) + (tid & 15) * 8;
  const bf16* vb = (tree_chunk ? vt_base : vc) + (tid & 15) * 8;
  auto load_kv = [&](int slot, int kt0) {
    int64_t base = (int64_t)kt0 * kst;
    if constexpr (PAGED) {
      if (!tree_chunk) {
        const CacheView cv{a.cb, a.ch, a.ct, a.table, a.ps, a.maxb, a.npages};
        bool ok;
        base = cache_offset(cv, b, 0, kt0, ok);  // kt0's slot in its page, head 0
      }
    }
    const int last = k1 - 1 - kt0;
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int r = min((tid + u * NWA * 64) >> 4, last);
      const int64_t off = base + (int64_t)r * kst;
      kreg[slot][u] = *(const uint4*)(kb + off);
      vreg[slot][u] = *(const uint4*)(vb + off);
    }
  };
  // ZERO: keys past the chunk end are stored as zeros.  They are masked to weight 0 either
  // way (and hold finite copies of the chunk's last key), so tiles that are full by
  // construction store the registers as they are.
  auto store_kv = [&](int slot, int buf, int kt0, auto ZC) {
    constexpr bool ZERO = decltype(ZC)::value;
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int i = tid + u * NWA * 64;
      const int kk = i >> 4, gd = i & 15;
      const bool ok = !ZERO || kt0 + kk < k1;
      *(uint4*)(ks[buf] + kk * KS + gd * 8) = ok ? kreg[slot][u] : make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)(vs[buf] + kk * VS + gd * 8) = ok ? vreg[slot][u] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  const int ntile = (k1 - k0 + KT - 1) / KT;
  load_kv(0, k0);
  load_kv(1, min(k0 + KT, k1 - 1));
  store_kv(0, 0, k0, std::true_type{});
  __syncthreads();
  // one tile: SL (compile-time, so the register ring never needs dynamic indexing) is the
  // register slot and LDS buffer of tile it.  MASKED: the tile has keys a row may not see
  // (tree keys, or keys past the chunk end); an unmasked tile (a full tile of prefix keys)
  // skips the visibility bits and scales each score inside the exponential's FMA.
  auto tile_step = [&](auto SLC, auto MC, int it) {
    constexpr int SL = decltype(SLC)::value;
    constexpr bool MASKED = decltype(MC)::value;
    const int kt0 = k0 + it * KT;
    // tile it + 2 into the slot tile it came through
    load_kv(SL, min(kt0 + 2 * KT, k1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    const bf16* ksb = ks[SL];
    const bf16* vsb = vs[SL];

    // visibility bits of this lane's 16 keys of the tile, per row block: the ancestor word
    // covering the tile (prefix chunks: all ones) cut at the chunk end, shifted to the lane's
    // 4-key group; key (st, i) is then bit (st & 1) * 16 + i of the low (st < 2) or high word
    uint32_t vlo[RBW], vhi[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      vlo[j] = vhi[j] = ~0u;
      if constexpr (MASKED) {
        // bits 0 .. n-1 set, n = the tile's keys before the chunk end, in [0, 64]; shift
        // arithmetic only (no select that could become a branch after the score MFMAs)
        const int n = min(max(k1 - kt0, 0), 64);
        const uint64_t bound = (~0ull >> ((64 - n) & 63)) & (0ull - (uint64_t)(n != 0));
        const uint64_t ws = (((kt0 & 64) ? vis1[j] : vis0[j]) & bound) >> (lq * 4);
        vlo[j] = (uint32_t)ws;
        vhi[j] = (uint32_t)(ws >> 32);
      }
    }
    // MASKED: scores in log2 units, -inf where hidden; unmasked: the raw q.k
    float s[RBW][4][4];
    // all 16 K fragments of the tile are requested before the first score MFMA, so the
    // LDS latency is paid once per tile rather than once per fragment
    bf16x8_t kf[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[st][kk] = *(const bf16x8_t*)(ksb + (st * 16 + lr) * KS + kk * 32 + lq * 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st][kk], qf[j][kk], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (MASKED) {
            const bool vis = ((st < 2 ? vlo[j] : vhi[j]) >> ((st & 1) * 16 + i)) & 1u;
            s[j][st][i] = vis ? acc[i] * sl2 : -INFINITY;
          } else {
            s[j][st][i] = acc[i];
          }
        }
      }
    }

#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][st][i]);
      mx = max_xor16_32(mx);
      if constexpr (!MASKED) mx *= sl2;  // sl2 > 0: the scaled maximum is the maximum scaled
      const float mnew = fmaxf(mrow[j], mx);
      const float mbase = (mnew == -INFINITY) ? 0.f : mnew;
      const float fac = __builtin_amdgcn_exp2f(mrow[j] - mbase);
      mrow[j] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = MASKED ? __builtin_amdgcn_exp2f(s[j][st][i] - mbase)
                                 : __builtin_amdgcn_exp2f(fmaf(s[j][st][i], sl2, -mbase));
          s[j][st][i] = p;
          ps += p;
        }
      lsum[j] = lsum[j] * fac + ps;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[j][db] *= fac;
    }

#pragma unroll
    for (int G = 0; G < 2; ++G) {
      bf16x8_t pb[RBW];
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        union {
          uint32_t u[4];
          bf16x8_t v;
        } pk;
        pk.u[0] = cvt_pk_bf16(s[j][2 * G][0], s[j][2 * G][1]);
        pk.u[1] = cvt_pk_bf16(s[j][2 * G][2], s[j][2 * G][3]);
        pk.u[2] = cvt_pk_bf16(s[j][2 * G + 1][0], s[j][2 * G + 1][1]);
        pk.u[3] = cvt_pk_bf16(s[j][2 * G + 1][2], s[j][2 * G + 1][3]);
        pb[j] = pk.v;
      }
      // V^T fragments by transpose reads: lane (q = lq, s = lr) addresses key
      // G*32 + 4q + s/4 (and + 16), d = db*16 + 4*(s%4)
      const bf16* vr = vsb + (G * 32 + 4 * lq + (lr >> 2)) * VS + 4 * (lr & 3);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        union {
          s16x4_t h[2];
          bf16x8_t v;
        } va;
        va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(vr + db * 16));
        va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vr + 16 * VS + db * 16));
#pragma unroll
        for (int j = 0; j < RBW; ++j) o[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb[j], o[j][db], 0, 0, 0);
      }
    }
    // next tile (loaded one step ago) into the other LDS buffer; the barrier also ends
    // every wave's reads of this buffer before it is refilled
    if (it + 1 < ntile) store_kv(1 - SL, 1 - SL, kt0 + KT, MC);
    __syncthreads();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // full prefix tiles (an even count, so every loop keeps the slot order) run unmasked;
  // the tree chunk's tiles and a prefix chunk's last tiles run masked
  const int nu = tree_chunk ? 0 : ((k1 - k0) / KT) & ~1;
  for (int it = 0; it < nu; it += 2) {
    tile_step(S0{}, Unmasked{}, it);
    tile_step(S1{}, Unmasked{}, it + 1);
  }
  for (int it = nu; it < ntile; it += 2) {
    tile_step(S0{}, Masked{}, it);
    if (it + 1 < ntile) tile_step(S1{}, Masked{}, it + 1);
  }

  const int rmax = a.max_nodes * g;
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    float l = lsum[j];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = row_base + (w * RBW + j) * 16 + lr;
    if (row < R) {
      const int64_t pidx = ((int64_t)(b * a.hkv + kvh) * a.n_chunks + c) * rmax + row;
      if (lq == 0) {
        a.part_ml[pidx * 2] = mrow[j];
        a.part_ml[pidx * 2 + 1] = l;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) *(f32x4*)(a.part_o + pidx * HD + db * 16 + lq * 4) = o[j][db];
    }
  }
}

// Combine the chunks of every query row in fixed order: o = sum_c 2^(m_c - M) o_c / L.
// A workgroup takes MROWS rows; 32 threads per row, each with 4 consecutive d (16-byte
// partial loads, one 8-byte bf16 store).  The partial loads do not wait for the prefix
// length: all MB chunks of a batch are loaded at once (clamped addresses, so they stay
// inside the workspace) and the chunks without data are dropped by selects afterwards, so
// a batch costs one round trip to memory.  MB is the smallest of 2, 4, 8, 12, 16 that covers
// the chunks (clamped duplicates would only add traffic); with more than 16 chunks the
// running (M, L, O) are rescaled between batches, otherwise the result is the two-pass
// one, bit for bit.
constexpr int MROWS = 8;
template <int MB>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int grid_real) {
  const int bid = blockIdx.x;
  if (bid >= grid_real) return;
  const int g = a.hq / a.hkv;
  const int rmax = a.max_nodes * g;
  const int rgroups = (rmax + MROWS - 1) / MROWS;
  int t = bid;
  const int rg = t % rgroups;
  t /= rgroups;
  const int kvh = t % a.hkv;
  const int b = t / a.hkv;
  const int row = rg * MROWS + threadIdx.x / 32;
  const int lrow = min(row, rmax - 1);  // address of the loads (rows past rmax exit below)
  const int d4 = (threadIdx.x % 32) * 4;
  const int nc = a.n_chunks;
  const int64_t base = (int64_t)(b * a.hkv + kvh) * nc;
  // scalars of the sequence (their loads overlap those of the first batch)
  const int off = a.tree_off[b];
  const int N = a.n_nodes ? a.n_nodes[b] : a.tree_off[b + 1] - off;
  const int qlo = a.q_lo ? a.q_lo[b] : 0;
  const int P = min(max(a.prefix_len[b], 0), a.cap);
  float M = -INFINITY, L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < nc; j0 += MB) {
    float2 ml[MB];
    float4 o4[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int64_t pi = (base + min(j0 + u, nc - 1)) * rmax + lrow;
      ml[u] = *(const float2*)(a.part_ml + pi * 2);
      o4[u] = *(const float4*)(a.part_o + pi * HD + d4);
    }
    // chunks with data: prefix chunks 0..n_pref-1, then the tree chunk (the last)
    const int n_pref = min((P + a.kch - 1) / a.kch, nc - 1);
    bool ok[MB];
    float mb = M;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int j = j0 + u;
      ok[u] = j < nc && (j < n_pref || j == nc - 1);
      mb = ok[u] ? fmaxf(mb, ml[u].x) : mb;
    }
    if (j0 > 0) {  // rescale what earlier batches summed (M = -inf: nothing summed yet)
      const float r = M > -INFINITY ? exp2f(M - mb) : 0.f;
      L *= r;
      O.x *= r;
      O.y *= r;
      O.z *= r;
      O.w *= r;
    }
    M = mb;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      if (!ok[u]) continue;
      const float f = exp2f(ml[u].x - M);
      L += f * ml[u].y;
      O.x += f * o4[u].x;
      O.y += f * o4[u].y;
      O.z += f * o4[u].z;
      O.w += f * o4[u].w;
    }
  }
  if (row >= (N - qlo) * g || N - qlo > a.max_nodes || N > 64 * a.mw) return;
  const float4 out = make_float4(O.x / L, O.y / L, O.z / L, O.w / L);
  const int node = qlo + row / g, hh = row % g;
  const int64_t orow = a.q_stride ? (int64_t)b * a.q_stride + (node - qlo) : (int64_t)(off + node);
  const int64_t oi = orow * a.hq * HD + (int64_t)(kvh * g + hh) * HD + d4;
  *(uint2*)((bf16*)a.out + oi) = make_uint2(cvt_pk_bf16(out.x, out.y), cvt_pk_bf16(out.z, out.w));
  if (a.dbg) *(float4*)(a.dbg + oi) = out;
}

// fp32 path: one workgroup per (sequence, query head, group of 8 nodes), one node per wave.
// Keys (the prefix, then the tree nodes) are taken in blocks of F32_KB: the block's K and V
// rows are staged in LDS with 16-byte loads by the whole workgroup; each wave then scores the
// block's keys for its node (a lane per key, dot products from LDS), folds the block into its
// running max and sum, and each lane accumulates output dimensions lane and lane + 64 from
// the V rows in LDS.  The LDS footprint does not depend on the prefix length.
constexpr int F32_KB = 128;   // keys per block
constexpr int F32_NG = 8;     // nodes (waves) per workgroup
constexpr int F32_KP = 132;   // LDS row stride (floats): 16-byte aligned rows
__global__ __launch_bounds__(F32_NG * 64) void tree_attn_f32_kernel(AttnArgs a, int groups) {
  __shared__ __align__(16) float ks[F32_KB * F32_KP];
  __shared__ __align__(16) float vs[F32_KB * F32_KP];
  __shared__ __align__(16) float qs[F32_NG][128];
  __shared__ float ps[F32_NG][F32_KB];
  const int hq = a.hq, hd = a.hd;
  int t = blockIdx.x;
  const int grp = t % groups;
  t /= groups;
  const int h = t % hq;
  const int b = t / hq;
  const int off = a.tree_off[b];
  const int N = a.tree_off[b + 1] - off;
  if (N > a.max_nodes || grp * F32_NG >= N) return;
  const int P = min(max(a.prefix_len[b], 0), a.cap);
  const int kvh = h / (hq / a.hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = grp * F32_NG + w;  // this wave's node
  const bool live = i < N;
  const int ic = live ? i : N - 1;
  const float* q = (const float*)a.q + ((int64_t)(off + ic) * hq + h) * hd;
  for (int d = lane; d < hd; d += 64) qs[w][d] = q[d];
  const uint64_t anc0 = a.anc[(int64_t)(off + ic) * a.mw];
  const uint64_t anc1 = a.mw > 1 ? a.anc[(int64_t)(off + ic) * a.mw + 1] : 0ull;
  const CacheView cv{a.cb, a.ch, a.ct, a.table, a.ps, a.maxb, a.npages};
  const float* kc = (const float*)a.k_cache;
  const float* vc = (const float*)a.v_cache;
  const float* ktr = (const float*)a.k_tree;
  const float* vtr = (const float*)a.v_tree;
  const float scale = rsqrtf((float)hd);
  const int c4 = hd / 4;  // 16-byte pieces per row
  float m = -INFINITY, l = 0.f;
  float acc[2] = {0.f, 0.f};
  for (int j0 = 0; j0 < P + N; j0 += F32_KB) {
    const int nb = min(F32_KB, P + N - j0);
    __syncthreads();  // the previous block's rows are no longer read
    for (int e = tid; e < nb * c4; e += blockDim.x) {
      const int r = e / c4, c = e % c4;
      const int j = j0 + r;
      int64_t ko;
      const float *kb, *vb;
      if (j < P) {
        bool ok;
        ko = cache_offset(cv, b, kvh, j, ok);
        kb = kc;
        vb = vc;
      } else {
        ko = ((int64_t)(off + j - P) * a.hkv + kvh) * hd;
        kb = ktr;
        vb = vtr;
      }
      *(float4*)&ks[r * F32_KP + 4 * c] = *(const float4*)(kb + ko + 4 * c);
      *(float4*)&vs[r * F32_KP + 4 * c] = *(const float4*)(vb + ko + 4 * c);
    }
    __syncthreads();
    if (live) {
      // scores of keys jj = lane and lane + 64 of the block
      float sc[2];
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int jj = lane + 64 * u;
        const int j = j0 + jj;
        bool vis = jj < nb;
        if (vis && j >= P) {
          const int jn = j - P;
          vis = (((jn < 64 ? anc0 : anc1) >> (jn & 63)) & 1ull) != 0ull;
        }
        float dot = 0.f;
        if (vis) {
          for (int d = 0; d < hd; d += 4) {
            const float4 kv = *(const float4*)&ks[jj * F32_KP + d];
            const float4 qv = *(const float4*)&qs[w][d];
            dot += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
          }
        }
        sc[u] = vis ? dot * scale : -INFINITY;
        bm = fmaxf(bm, sc[u]);
      }
      bm = wave_max(bm);
      const float mnew = fmaxf(m, bm);
      if (mnew != -INFINITY) {  // else every key so far is hidden: nothing to add
        const float fac = m == -INFINITY ? 0.f : __expf(m - mnew);
        float bs = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float pu = __expf(sc[u] - mnew);
          ps[w][lane + 64 * u] = pu;
          bs += pu;
        }
        l = l * fac + wave_sum(bs);
        acc[0] *= fac;
        acc[1] *= fac;
        m = mnew;
        __builtin_amdgcn_wave_barrier();
        for (int jj = 0; jj < nb; ++jj) {
          const float pj = ps[w][jj];
          acc[0] += pj * vs[jj * F32_KP + lane];
          if (lane + 64 < hd) acc[1] += pj * vs[jj * F32_KP + lane + 64];
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (!live) return;
  for (int u = 0; u < 2; ++u) {
    const int d = lane + 64 * u;
    if (d >= hd) break;
    const float out = acc[u] / l;
    const int64_t oi = (int64_t)(off + i) * hq * hd + (int64_t)h * hd + d;
    ((float*)a.out)[oi] = out;
    if (a.dbg) a.dbg[oi] = out;
  }
}

}  // namespace

AttnPlan plan_attn(int dtype, int batch, int hq, int hkv, int hd, int max_nodes, int max_prefix) {
  AttnPlan p{};
  const int g = hq / hkv;
  p.rmax = max_nodes * g;
  if (dtype == EAGLE_F32) {
    p.kch = 0;
    p.n_chunks = 0;
    p.row_groups = 0;
    return p;
  }
  // prefix chunks: about 512 (b, kv head, chunk, row group) workgroups, with at least 256
  // keys and at most 32 chunks per (b, kv head)
  auto chunks = [&](int nwa) {
    p.nwa = nwa;
    p.row_groups = (p.rmax + nwa * 16 - 1) / (nwa * 16);
    const int units = std::max(1, batch * hkv * p.row_groups);
    int nch = std::max(1, (512 + units - 1) / units);
    nch = std::min(nch, std::max(1, (max_prefix + 255) / 256));
    nch = std::min(nch, 32);
    int kch = (max_prefix + nch - 1) / nch;
    kch = std::max(KT, (kch + KT - 1) / KT * KT);
    nch = std::max(1, (max_prefix + kch - 1) / kch);
    p.kch = kch;
    p.n_chunks = nch + 1;  // + the tree chunk
    return units * p.n_chunks;
  };
  // Four-wave workgroups (64 query rows, two per CU) when a (b, kv head) pair has at most
  // 64 query rows, or when eight-wave ones would not cover the CUs once: the draft's levels
  // (16 sequences x 40 rows per kv head) measured 12% faster and one 60-node tree at
  // prefix 2048 9% faster; where eight-wave workgroups fill the chip (hundreds of rows per
  // pair, or many sequences) four-wave ones were 8-10% slower, since each row group
  // re-reads its chunk's keys.
  if (p.rmax <= 64 || chunks(8) < 256) chunks(4);
  (void)hd;
  return p;
}

size_t attn_workspace_floats(const AttnPlan& p, int batch, int hkv, int hd) {
  if (p.n_chunks == 0) return 0;
  const size_t rows = (size_t)batch * hkv * p.n_chunks * p.rmax;
  return rows * hd + rows * 2;
}

int launch_attn(AttnArgs& a, const AttnPlan& p, eagle_timer* timer, hipStream_t s) {
  if (a.dtype == EAGLE_F32) return EAGLE_ERR_ARG;  // the fp32 path is launch_attn_f32
  if (a.hd != HD) return EAGLE_ERR_UNSUPPORTED;
  a.kch = p.kch;
  a.n_chunks = p.n_chunks;
  a.row_groups = p.row_groups;
  const int grid = a.batch * a.hkv * p.n_chunks * p.row_groups;
  const int padded = (grid + kXcds - 1) / kXcds * kXcds;
  timer_begin(timer, ST_ATTN, s);
  if (p.nwa == 4) {
    if (a.table)
      hipLaunchKernelGGL((tree_attn_bf16_kernel<4, true>), dim3(padded), dim3(4 * 64), 0, s, a, grid);
    else
      hipLaunchKernelGGL((tree_attn_bf16_kernel<4, false>), dim3(padded), dim3(4 * 64), 0, s, a, grid);
  } else if (p.nwa == 8) {
    if (a.table)
      hipLaunchKernelGGL((tree_attn_bf16_kernel<8, true>), dim3(padded), dim3(8 * 64), 0, s, a, grid);
    else
      hipLaunchKernelGGL((tree_attn_bf16_kernel<8, false>), dim3(padded), dim3(8 * 64), 0, s, a, grid);
  } else {
    return EAGLE_ERR_UNSUPPORTED;
  }
  timer_end(timer, s);
  const int g = a.hq / a.hkv;
  const int mgrid = a.batch * a.hkv * ((a.max_nodes * g + MROWS - 1) / MROWS);
  timer_begin(timer, ST_ATTN_MERGE, s);
  if (p.n_chunks <= 2)
    hipLaunchKernelGGL(attn_merge_kernel<2>, dim3(mgrid), dim3(256), 0, s, a, mgrid);
  else if (p.n_chunks <= 4)
    hipLaunchKernelGGL(attn_merge_kernel<4>, dim3(mgrid), dim3(256), 0, s, a, mgrid);
  else if (p.n_chunks <= 8)
    hipLaunchKernelGGL(attn_merge_kernel<8>, dim3(mgrid), dim3(256), 0, s, a, mgrid);
  else if (p.n_chunks <= 12)
    hipLaunchKernelGGL(attn_merge_kernel<12>, dim3(mgrid), dim3(256), 0, s, a, mgrid);
  else
    hipLaunchKernelGGL(attn_merge_kernel<16>, dim3(mgrid), dim3(256), 0, s, a, mgrid);
  timer_end(timer, s);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_attn_f32(AttnArgs& a, int total_nodes, eagle_timer* timer, hipStream_t s) {
  (void)total_nodes;
  if (a.hd != 64 && a.hd != 128) return EAGLE_ERR_UNSUPPORTED;
  if ((a.cb | a.ch | a.ct) % 4) return EAGLE_ERR_ARG;  // rows are read with 16-byte loads
  const int groups = (a.max_nodes + F32_NG - 1) / F32_NG;
  timer_begin(timer, ST_ATTN, s);
  hipLaunchKernelGGL(tree_attn_f32_kernel, dim3(a.batch * a.hq * groups), dim3(F32_NG * 64), 0, s, a, groups);
  timer_end(timer, s);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle
