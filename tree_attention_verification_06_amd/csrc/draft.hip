// Draft-head tree expansion (EAGLE feature-level drafting with EAGLE-2-style pruning).
//
// Level-synchronous and entirely on the device (no host synchronisation).  Level l
// expands the frontier of every sequence as one batch of token rows, row r = b * FL + j
// (FL = 1 on the first level, the frontier width afterwards; rows of a sequence beyond
// its frontier are padding, computed but never read back):
//   prep     frontier -> row inputs (parent feature row, token, position), a K/V slot
//            and an ancestor word over the expanded nodes of the sequence
//   FC       x = W_fc [f_parent ; E[token]]  (both halves gathered by the GEMM prologue)
//   layer    RMSNorm -> QKV + rotary -> tree attention over [draft KV prefix ; expanded
//            nodes on the row's root path] -> O + residual -> RMSNorm -> gate/up ->
//            down + residual = predicted feature f_hat
//   LM head  the target's head on RMSNorm(f_hat); its epilogue keeps each tile's top-k
//            (value, id) and (max, sum exp) per row, so no logits reach HBM
//   merge    per row: top-k over the tiles (ties to the lower id) and the log-sum-exp
//   select   per sequence: children, cum = cum(parent) + min(0, log p), expandable iff
//            log p >= log(threshold), next frontier = the best `frontier` expandable
//            children by (cum desc, generation order asc)
// and rerank keeps the root plus the best max_nodes-1 candidates by (cum desc, depth asc,
// generation asc), re-indexed by (depth asc, cum desc, generation asc).
//
// Candidates live in a per-sequence pool in generation order: root, then the children of
// each level in (parent frontier rank, child rank) order.  Depth equals the level, so
// pool order is (depth, generation order) and every ordering above is an exact 64-bit
// key comparison; ranks are counted in LDS (no data-dependent sorting network).
#include <algorithm>
#include <cmath>

#include "attn.h"
#include "draft.h"
#include "gemm.h"

namespace eagle {

namespace {

constexpr int POOL_MAX = 2048;  // candidates per sequence
constexpr int KMAX = 16;        // top_k and frontier limit
constexpr int MAXP = 64;        // expanded nodes per sequence (one ancestor word)

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PoolRec {
  int32_t token, parent, depth, slot;
  float cum, logp;
};

// per-sequence counters, stored as [field][B]
enum { C_NNODES = 0, C_QLO = 1, C_NF = 2, C_POOLN = 3, C_FIELDS = 4 };

struct DraftLayout {
  int maxp, pool;
  GemmPlan p_fc[2], p_qkv[2], p_o[2], p_gu[2], p_down[2], p_lm[2];  // [0]: first level, [1]: later levels
  AttnPlan pa[2];
  size_t feat, x, x16, ssq_x, q, kd, vd, anc, att, attn_part, y, y16, ssq_y, act, h, h16, ssq_h;
  size_t tk_val, tk_idx, tk_lse, row_val, row_idx, row_lse, rows, cnt, att_off, pool_recs, frontier, lvl_front;
  size_t gpart, gssq, counters, total;
  int n_tk_max;
};

DraftLayout plan_draft(const eagle_dims* d, const eagle_draft_params* pr, int B, int max_prefix) {
  DraftLayout L{};
  const int F = pr->frontier, K = pr->top_k;
  L.maxp = 1 + (pr->depth - 1) * F;
  L.pool = 1 + K + (pr->depth - 1) * F * K;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, Dh = d->head_dim, Fm = d->ffn, V = d->vocab;
  const int R = B * F;
  size_t pf = 0, sf = 0, ci = 0;
  int nt_max = 1;
  L.n_tk_max = 1;
  for (int i = 0; i < 2; ++i) {
    const int m = i == 0 ? B : R;
    L.p_fc[i] = plan_gemm(EAGLE_BF16, H, 2 * H, m, 0, EPI_RESID, Dh);
    L.p_qkv[i] = plan_gemm(EAGLE_BF16, (Hq + 2 * Hkv) * Dh, H, m, 0, EPI_QKV, Dh);
    L.p_o[i] = plan_gemm(EAGLE_BF16, H, Hq * Dh, m, 0, EPI_RESID, Dh);
    L.p_gu[i] = plan_gemm(EAGLE_BF16, Fm, H, m, 1, EPI_SILU, Dh);
    L.p_down[i] = plan_gemm(EAGLE_BF16, H, Fm, m, 0, EPI_RESID, Dh);
    L.p_lm[i] = plan_gemm(EAGLE_BF16, V, H, m, 0, EPI_TOPK, Dh);
    L.pa[i] = plan_attn(EAGLE_BF16, B, Hq, Hkv, Dh, i == 0 ? 1 : F, max_prefix);
    for (const GemmPlan* p : {&L.p_fc[i], &L.p_qkv[i], &L.p_o[i], &L.p_gu[i], &L.p_down[i], &L.p_lm[i]}) {
      size_t a, b2, c;
      gemm_workspace(*p, &a, &b2, &c);
      pf = std::max(pf, a);
      sf = std::max(sf, b2);
      ci = std::max(ci, c);
    }
    nt_max = std::max({nt_max, L.p_fc[i].n_tiles, L.p_o[i].n_tiles, L.p_down[i].n_tiles});
    L.n_tk_max = std::max(L.n_tk_max, L.p_lm[i].n_tiles);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(std::max<size_t>(bytes, 1));
    return o;
  };
  L.feat = take((size_t)(B + B * L.maxp) * H * 2);  // bf16 rows: B root features, then B x maxp slots
  L.x = take((size_t)R * H * 4);
  L.x16 = take((size_t)R * H * 2);
  L.ssq_x = take((size_t)nt_max * R * 4);
  L.q = take((size_t)R * Hq * Dh * 2);
  L.kd = take((size_t)B * L.maxp * Hkv * Dh * 2);
  L.vd = take((size_t)B * L.maxp * Hkv * Dh * 2);
  L.anc = take((size_t)B * L.maxp * 8);
  L.att = take((size_t)R * Hq * Dh * 2);
  L.attn_part =
      take(std::max(attn_workspace_floats(L.pa[0], B, Hkv, Dh), attn_workspace_floats(L.pa[1], B, Hkv, Dh)) * 4);
  L.y = take((size_t)R * H * 4);
  L.y16 = take((size_t)R * H * 2);
  L.ssq_y = take((size_t)nt_max * R * 4);
  L.act = take((size_t)R * Fm * 2);
  L.h = take((size_t)R * H * 4);
  L.h16 = take((size_t)R * H * 2);
  L.ssq_h = take((size_t)nt_max * R * 4);
  L.tk_val = take((size_t)R * L.n_tk_max * K * 4);
  L.tk_idx = take((size_t)R * L.n_tk_max * K * 4);
  L.tk_lse = take((size_t)R * L.n_tk_max * 2 * 4);
  L.row_val = take((size_t)R * K * 4);
  L.row_idx = take((size_t)R * K * 4);
  L.row_lse = take((size_t)R * 4);
  L.rows = take((size_t)R * 4 * 4);  // feat_idx | tok | pos | kv_idx
  L.cnt = take((size_t)C_FIELDS * B * 4);
  L.att_off = take((size_t)(B + 1) * 4);
  L.pool_recs = take((size_t)B * L.pool * sizeof(PoolRec));
  L.frontier = take((size_t)B * F * 4);
  L.lvl_front = take((size_t)B * pr->depth * F * 4);
  L.gpart = take(pf * 4);
  L.gssq = take(sf * 4);
  L.counters = take(ci * 4);
  L.total = off;
  return L;
}

struct DraftState {
  int B, H, F, K, M, maxp, pool, depth, level, FL, FLprev, n_tk;
  float log_tau;  // log(threshold); -inf: no pruning
  const int32_t* prefix_len;
  const int32_t* root_token;
  const float* root_feature;
  bf16* feat;
  const float* h;  // predicted features of the previous level [B * FLprev][H] (level > 1)
  int32_t *feat_idx, *tok, *pos, *kv_idx;
  int32_t* cnt;
  int32_t* att_off;
  PoolRec* pool_recs;
  int32_t* frontier;
  int32_t* lvl_front;
  uint64_t* anc;
  const float* tk_val;
  const int32_t* tk_idx;
  const float* tk_lse;
  float* row_val;
  int32_t* row_idx;
  float* row_lse;
};

// -0 and +0 compare equal but map to different ordered keys; cum values are kept at +0
__device__ __forceinline__ float canon_zero(float v) { return v == 0.f ? 0.f : v; }

// Root features to bf16, pool = {root}, frontier = {root}, attention tree offsets b * maxp.
__global__ __launch_bounds__(256) void draft_init_kernel(DraftState s) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x * 4; i < s.H; i += blockDim.x * 4) {
    const float4 v = *(const float4*)(s.root_feature + (int64_t)b * s.H + i);
    *(uint2*)(s.feat + (int64_t)b * s.H + i) = make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
  }
  if (threadIdx.x == 0) {
    PoolRec r;
    r.token = s.root_token[b];
    r.parent = -1;
    r.depth = 0;
    r.slot = -1;
    r.cum = 0.f;
    r.logp = 0.f;
    s.pool_recs[(int64_t)b * s.pool] = r;
    s.frontier[(int64_t)b * s.F] = 0;
    s.cnt[C_NNODES * s.B + b] = 0;
    s.cnt[C_QLO * s.B + b] = 0;
    s.cnt[C_NF * s.B + b] = 1;
    s.cnt[C_POOLN * s.B + b] = 1;
    s.att_off[b] = b * s.maxp;
    if (b == s.B - 1) s.att_off[s.B] = s.B * s.maxp;
  }
  for (int i = threadIdx.x; i < s.depth * s.F; i += blockDim.x) s.lvl_front[(int64_t)b * s.depth * s.F + i] = -1;
}

// Frontier of sequence b -> rows b*FL .. b*FL+FL-1.  Also stores the previous level's
// predicted features (bf16) in the feature rows of the nodes expanded there.
// Workgroup (b, 0) does the bookkeeping; workgroup (b, 1 + j) copies row j of the previous
// level (one feature row each, so the copy runs on B * FLprev workgroups).
__global__ __launch_bounds__(256) void draft_prep_kernel(DraftState s) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int m0 = s.cnt[C_NNODES * s.B + b];  // nodes expanded before this level
  const int qlo_prev = s.cnt[C_QLO * s.B + b];
  const int nf = s.cnt[C_NF * s.B + b];
  if (blockIdx.y > 0) {
    const int j = blockIdx.y - 1;
    if (!s.h || j >= m0 - qlo_prev) return;  // nodes expanded on the previous level: slots qlo_prev ..
    const int64_t frow = (int64_t)s.B + (int64_t)b * s.maxp + qlo_prev + j;
    for (int c = tid * 4; c < s.H; c += blockDim.x * 4) {
      const float4 v = *(const float4*)(s.h + ((int64_t)b * s.FLprev + j) * s.H + c);
      *(uint2*)(s.feat + frow * s.H + c) = make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
    }
    return;
  }
  if (tid < s.FL) {
    const int j = tid, r = b * s.FL + j;
    if (j < nf) {
      PoolRec* pr = s.pool_recs + (int64_t)b * s.pool;
      const int node = s.frontier[(int64_t)b * s.F + j];
      const int par = pr[node].parent;
      const int slot = m0 + j;
      const int pslot = par < 0 ? -1 : pr[par].slot;
      pr[node].slot = slot;
      const uint64_t w = (pslot < 0 ? 0ull : s.anc[(int64_t)b * s.maxp + pslot]) | (1ull << slot);
      s.anc[(int64_t)b * s.maxp + slot] = w;
      s.feat_idx[r] = pslot < 0 ? b : s.B + b * s.maxp + pslot;
      s.tok[r] = pr[node].token;
      s.pos[r] = s.prefix_len[b] + pr[node].depth;
      s.kv_idx[r] = b * s.maxp + slot;
      s.lvl_front[((int64_t)b * s.depth + (s.level - 1)) * s.F + j] = node;
    } else {
      s.feat_idx[r] = b;
      s.tok[r] = 0;
      s.pos[r] = 0;
      s.kv_idx[r] = -1;
    }
  }
  __syncthreads();
  if (tid == 0) {
    s.cnt[C_QLO * s.B + b] = m0;
    s.cnt[C_NNODES * s.B + b] = m0 + nf;
  }
}

// Row top-k over the LM-head tiles (ties to the lower id) and the row log-sum-exp.
// Each thread keeps a sorted list of its best KMAX candidates (branch-free insertion,
// static indices); each wave then selects its top K from its lanes' lists, and one
// thread merges the four wave lists.
// KL: length of the per-thread candidate lists (>= K): the sorted insertion costs KL steps.
template <int KL>
__global__ __launch_bounds__(256) void draft_topk_merge_kernel(DraftState s) {
  const int r = blockIdx.x;
  const int b = r / s.FL, j = r % s.FL;
  if (j >= s.cnt[C_NF * s.B + b]) return;
  __shared__ float fred[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // per-tile outputs are stored row-major: [row][tile][...], so this row's are contiguous
  const float* lp = s.tk_lse + (int64_t)r * s.n_tk * 2;
  const int64_t ls = 2;
  // one pass over the tiles' (max, sum) pairs, 4 loads per thread per round (clamped,
  // unconditional), summed with a running maximum; waves, then the workgroup, combine their
  // (max, sum) pairs the same way
  const int nth = blockDim.x;
  float mx = -INFINITY, se = 0.f;
  for (int t0 = tid; t0 < s.n_tk; t0 += 4 * nth) {
    float m4[4], s4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t o = (int64_t)min(t0 + u * nth, s.n_tk - 1) * ls;
      m4[u] = lp[o];
      s4[u] = lp[o + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = t0 + u * nth < s.n_tk && m4[u] > -INFINITY;
      const float mn = ok ? fmaxf(mx, m4[u]) : mx;
      const float add = ok ? s4[u] * __expf(m4[u] - mn) : 0.f;
      se = (mx > -INFINITY ? se * __expf(mx - mn) : 0.f) + add;
      mx = mn;
    }
  }
  const float wm = wave_max(mx);
  se = wave_sum(mx > -INFINITY ? se * __expf(mx - wm) : 0.f);
  __shared__ float fsum[4];
  if (lane == 0) {
    fred[w] = wm;
    fsum[w] = se;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) S += fred[i] > -INFINITY ? fsum[i] * __expf(fred[i] - M) : 0.f;
  const float lse = M + __logf(S);

  // candidate keys as doubles (see topk_key): one v_max_f64 / v_min_f64 pair per
  // insertion step, and a wave maximum that stays in the VALU
  double lst[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) lst[i] = 0.0;
  // the row's n_tk * K candidates are contiguous: thread tid takes candidates tid, tid +
  // 256, ... (coalesced), CU of them per round with unconditional, clamped loads (a
  // candidate past the end repeats the last one and is dropped, inserting the empty key 0)
  constexpr int CU = 16;
  const int64_t ob = (int64_t)r * s.n_tk * s.K;
  const int ne = s.n_tk * s.K;
  for (int e0 = tid; e0 < ne; e0 += CU * nth) {
    float vv[CU];
    int ii[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int64_t o = ob + min(e0 + u * nth, ne - 1);
      vv[u] = s.tk_val[o];
      ii[u] = s.tk_idx[o];
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      double key = (e0 + u * nth < ne && ii[u] >= 0) ? topk_key(vv[u], (uint32_t)ii[u]) : 0.0;
#pragma unroll
      for (int i = 0; i < KL; ++i) topk_cas(key, lst[i]);
    }
  }
  // each wave: K rounds of a wave maximum over its lanes' list heads (no barriers); the
  // winner pops its head (keys are unique: one per vocabulary id)
  __shared__ unsigned long long wtop[4][KMAX];
  for (int q = 0; q < s.K; ++q) {
    const double best = wave_max_key(lst[0]);
    if (best != 0.0 && lst[0] == best) {  // keys are unique: one lane pops its head
#pragma unroll
      for (int i = 0; i < KL - 1; ++i) lst[i] = lst[i + 1];
      lst[KL - 1] = 0.0;
    }
    if (lane == 0) wtop[w][q] = (unsigned long long)__double_as_longlong(best);
  }
  __syncthreads();
  if (tid == 0) {
    // 4-way merge of the wave lists
    int head[4] = {0, 0, 0, 0};
    for (int q = 0; q < s.K; ++q) {
      unsigned long long best = 0ull;
      int bw = 0;
      for (int i = 0; i < 4; ++i) {
        const unsigned long long c = head[i] < s.K ? wtop[i][head[i]] : 0ull;
        if (c > best) {
          best = c;
          bw = i;
        }
      }
      if (best != 0ull) head[bw]++;
      const bool ok = best != 0ull;
      s.row_val[(int64_t)r * s.K + q] = ok ? topk_key_value(best) : -INFINITY;
      s.row_idx[(int64_t)r * s.K + q] = ok ? topk_key_col(best) : -1;
    }
    s.row_lse[r] = lse;
  }
}

// Children of this level's frontier are appended to the pool; the next frontier is the
// best `frontier` expandable children.  One workgroup per sequence, one thread per child.
__global__ __launch_bounds__(256) void draft_select_kernel(DraftState s) {
  const int b = blockIdx.x, c = threadIdx.x;
  const int nf = s.cnt[C_NF * s.B + b];
  const int base = s.cnt[C_POOLN * s.B + b];
  PoolRec* pr = s.pool_recs + (int64_t)b * s.pool;
  __shared__ unsigned long long keys[256];
  __shared__ int sel[KMAX];
  const int nch = nf * s.K;
  unsigned long long key = 0ull;
  if (c < nch) {
    const int j = c / s.K, k = c % s.K;
    const int r = b * s.FL + j;
    const int node = s.frontier[(int64_t)b * s.F + j];
    const int tok = s.row_idx[(int64_t)r * s.K + k];
    const float logp = s.row_val[(int64_t)r * s.K + k] - s.row_lse[r];
    PoolRec rec;
    rec.token = tok;
    rec.parent = node;
    rec.depth = pr[node].depth + 1;
    rec.slot = -1;
    rec.cum = canon_zero(pr[node].cum + fminf(0.f, logp));
    rec.logp = logp;
    pr[base + c] = rec;
    if (tok >= 0 && logp >= s.log_tau)
      key = ((unsigned long long)f2ord(rec.cum) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)(base + c));
  }
  keys[c] = key;
  const int n_exp = __syncthreads_count(key != 0ull);
  if (key != 0ull) {
    int rank = 0;
    for (int i = 0; i < nch; ++i) rank += keys[i] > key;
    if (rank < s.F) sel[rank] = base + c;
  }
  __syncthreads();
  const int n = min(n_exp, s.F);
  if (c < s.F) s.frontier[(int64_t)b * s.F + c] = c < n ? sel[c] : -1;
  if (c == 0) {
    s.cnt[C_NF * s.B + b] = n;
    s.cnt[C_POOLN * s.B + b] = base + nch;
  }
}

// Final tree of sequence b, written at its offset in the compacted outputs.
__global__ __launch_bounds__(256) void draft_rerank_kernel(DraftState s, int32_t* tree_off, int32_t* parent,
                                                           int32_t* tokens, float* cum_out) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ unsigned long long k1[POOL_MAX];
  __shared__ float s_cum[POOL_MAX];
  __shared__ int s_dep[POOL_MAX], s_par[POOL_MAX], s_tok[POOL_MAX], newidx[POOL_MAX];
  __shared__ int kept[128], order[128];
  __shared__ unsigned long long k2[128];
  const int pn = s.cnt[C_POOLN * s.B + b];
  int off = 0;
  for (int i = 0; i < b; ++i) off += min(s.M, s.cnt[C_POOLN * s.B + i]);
  const int keep = min(s.M - 1, pn - 1);
  const PoolRec* pr = s.pool_recs + (int64_t)b * s.pool;
  for (int i = tid; i < pn; i += blockDim.x) {
    const PoolRec r = pr[i];
    s_cum[i] = r.cum;
    s_dep[i] = r.depth;
    s_par[i] = r.parent;
    s_tok[i] = r.token;
    newidx[i] = -1;
    k1[i] = i == 0 ? 0ull : ((unsigned long long)f2ord(r.cum) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
  }
  __syncthreads();
  // kept candidates: rank by (cum desc, pool order asc) below keep
  for (int i = 1 + tid; i < pn; i += blockDim.x) {
    const unsigned long long key = k1[i];
    int rank = 0;
    for (int q = 1; q < pn; ++q) rank += k1[q] > key;
    if (rank < keep) kept[rank] = i;
  }
  __syncthreads();
  // re-index: (depth asc, cum desc, pool order asc)
  for (int i = tid; i < keep; i += blockDim.x) {
    const int id = kept[i];
    k2[i] = ((unsigned long long)(63 - s_dep[id]) << 48) | ((unsigned long long)f2ord(s_cum[id]) << 16) |
            (unsigned long long)(0xffffu - (uint32_t)id);
  }
  __syncthreads();
  for (int i = tid; i < keep; i += blockDim.x) {
    const unsigned long long key = k2[i];
    int rank = 0;
    for (int q = 0; q < keep; ++q) rank += k2[q] > key;
    newidx[kept[i]] = 1 + rank;
    order[1 + rank] = kept[i];
  }
  if (tid == 0) {
    newidx[0] = 0;
    order[0] = 0;
  }
  __syncthreads();
  for (int i = tid; i <= keep; i += blockDim.x) {
    const int id = order[i];
    parent[off + i] = i == 0 ? -1 : newidx[s_par[id]];
    tokens[off + i] = s_tok[id];
    cum_out[off + i] = s_cum[id];
  }
  if (tid == 0) tree_off[b] = off;
  if (b == s.B - 1) {
    // entries past the last tree (pruned trees are shorter) are inert padding
    const int end = off + keep + 1;
    if (tid == 0) tree_off[s.B] = end;
    for (int i = end + tid; i < s.B * s.M; i += blockDim.x) {
      parent[i] = -1;
      tokens[i] = 0;
      cum_out[i] = -INFINITY;
    }
  }
}

// Candidate pool of the last expansion, structure of arrays.
__global__ __launch_bounds__(256) void draft_pool_kernel(DraftState s, int32_t* pool_n, int32_t* token,
                                                         int32_t* parent, int32_t* depth, float* cum, float* logp,
                                                         int32_t* expanded) {
  const int b = blockIdx.x;
  const int pn = s.cnt[C_POOLN * s.B + b];
  const PoolRec* pr = s.pool_recs + (int64_t)b * s.pool;
  for (int i = threadIdx.x; i < s.pool; i += blockDim.x) {
    const int64_t o = (int64_t)b * s.pool + i;
    const bool v = i < pn;
    const PoolRec r = pr[v ? i : 0];
    if (token) token[o] = v ? r.token : -1;
    if (parent) parent[o] = v ? r.parent : -1;
    if (depth) depth[o] = v ? r.depth : -1;
    if (cum) cum[o] = v ? r.cum : -INFINITY;
    if (logp) logp[o] = v ? r.logp : -INFINITY;
  }
  if (expanded)
    for (int i = threadIdx.x; i < s.depth * s.F; i += blockDim.x)
      expanded[(int64_t)b * s.depth * s.F + i] = s.lvl_front[(int64_t)b * s.depth * s.F + i];
  if (threadIdx.x == 0 && pool_n) pool_n[b] = pn;
}

int check_draft(const eagle_dims* d, const eagle_draft_params* p, int B, int max_prefix) {
  if (!d || !p || B < 1 || max_prefix < 0) return EAGLE_ERR_ARG;
  if (d->dtype != EAGLE_BF16 || d->head_dim != 128 || d->ffn <= 0 || d->rms_eps <= 0.f) return EAGLE_ERR_UNSUPPORTED;
  if (d->hidden <= 0 || d->hidden % 64 || d->ffn % 64 || d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads ||
      d->vocab < 1)
    return EAGLE_ERR_UNSUPPORTED;
  if (p->depth < 1 || p->top_k < 1 || p->top_k > KMAX || p->top_k > d->vocab || p->frontier < 1 ||
      p->frontier > KMAX || p->max_nodes < 2 || p->max_nodes > 128)
    return EAGLE_ERR_UNSUPPORTED;
  if (1 + (p->depth - 1) * p->frontier > MAXP) return EAGLE_ERR_UNSUPPORTED;
  if (1 + p->top_k + (p->depth - 1) * p->frontier * p->top_k > POOL_MAX) return EAGLE_ERR_UNSUPPORTED;
  if (p->frontier * p->top_k > 256) return EAGLE_ERR_UNSUPPORTED;
  if (!(p->conf_threshold >= 0.f && p->conf_threshold <= 1.f)) return EAGLE_ERR_ARG;
  if (d->lm_layout != 0 && d->lm_layout != 1) return EAGLE_ERR_ARG;
  return EAGLE_OK;
}

DraftState make_state(const DraftLayout& L, const eagle_dims* d, const eagle_draft_params* pr, int B, char* w) {
  DraftState st{};
  st.B = B;
  st.H = d->hidden;
  st.F = pr->frontier;
  st.K = pr->top_k;
  st.M = pr->max_nodes;
  st.maxp = L.maxp;
  st.pool = L.pool;
  st.depth = pr->depth;
  st.log_tau = pr->conf_threshold > 0.f ? std::log(pr->conf_threshold) : -INFINITY;
  st.feat = (bf16*)(w + L.feat);
  const int R = B * pr->frontier;
  int32_t* rows = (int32_t*)(w + L.rows);
  st.feat_idx = rows;
  st.tok = rows + R;
  st.pos = rows + 2 * R;
  st.kv_idx = rows + 3 * R;
  st.cnt = (int32_t*)(w + L.cnt);
  st.att_off = (int32_t*)(w + L.att_off);
  st.pool_recs = (PoolRec*)(w + L.pool_recs);
  st.frontier = (int32_t*)(w + L.frontier);
  st.lvl_front = (int32_t*)(w + L.lvl_front);
  st.anc = (uint64_t*)(w + L.anc);
  st.tk_val = (const float*)(w + L.tk_val);
  st.tk_idx = (const int32_t*)(w + L.tk_idx);
  st.tk_lse = (const float*)(w + L.tk_lse);
  st.row_val = (float*)(w + L.row_val);
  st.row_idx = (int32_t*)(w + L.row_idx);
  st.row_lse = (float*)(w + L.row_lse);
  return st;
}

XSeg bseg(const void* p, int64_t ld, const int32_t* idx) {
  XSeg sg;
  sg.ptr = p;
  sg.dtype = EAGLE_BF16;
  sg.ld = ld;
  sg.idx = idx;
  return sg;
}

}  // namespace

size_t draft_workspace(const eagle_dims* d, const eagle_draft_params* p, int batch, int max_prefix) {
  if (check_draft(d, p, batch, max_prefix)) return 0;
  return plan_draft(d, p, batch, max_prefix).total;
}

int draft_expand_impl(const eagle_dims* d, const eagle_draft_params* pr, const void* w_fc, const eagle_layer_w* lw,
                      const void* final_ln, const void* w_lm, const void* embed, int B, const float* root_feature,
                      const int32_t* root_token, const void* dk_cache, const void* dv_cache,
                      const eagle_cache_layout* cache, const int32_t* prefix_len, int max_prefix, int32_t* tree_off,
                      int32_t* parent, int32_t* tokens, float* cum_logp, void* ws, size_t ws_bytes,
                      eagle_timer* timer, hipStream_t s) {
  int rc = check_draft(d, pr, B, max_prefix);
  if (rc) return rc;
  if (!w_fc || !lw || !final_ln || !w_lm || !embed || !root_feature || !root_token || !dk_cache || !dv_cache ||
      !cache || !prefix_len || !tree_off || !parent || !tokens || !cum_logp || !ws)
    return EAGLE_ERR_ARG;
  if (!lw->ln_attn || !lw->w_qkv || !lw->w_o || !lw->ln_mlp || !lw->w_gate || !lw->w_up || !lw->w_down)
    return EAGLE_ERR_ARG;
  if (lw->layout != 0 && lw->layout != 1) return EAGLE_ERR_ARG;
  if (((uintptr_t)ws) & 255) return EAGLE_ERR_ARG;
  if (check_cache_layout(cache)) return EAGLE_ERR_ARG;
  const DraftLayout L = plan_draft(d, pr, B, max_prefix);
  if (ws_bytes < L.total) return EAGLE_ERR_WORKSPACE;
  char* w = (char*)ws;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, Dh = d->head_dim, Fm = d->ffn, V = d->vocab;
  const int F = pr->frontier, K = pr->top_k;
  DraftState st = make_state(L, d, pr, B, w);
  st.prefix_len = prefix_len;
  st.root_token = root_token;
  st.root_feature = root_feature;

  float* x = (float*)(w + L.x);
  void* x16 = w + L.x16;
  float* ssq_x = (float*)(w + L.ssq_x);
  void* qb = w + L.q;
  void* kd = w + L.kd;
  void* vd = w + L.vd;
  void* att = w + L.att;
  float* y = (float*)(w + L.y);
  void* y16 = w + L.y16;
  float* ssq_y = (float*)(w + L.ssq_y);
  void* act = w + L.act;
  float* h = (float*)(w + L.h);
  void* h16 = w + L.h16;
  float* ssq_h = (float*)(w + L.ssq_h);
  auto gemm = [&](GemmDesc& g, const GemmPlan& p, int stage) {
    g.dtype = EAGLE_BF16;
    g.partials = (float*)(w + L.gpart);
    g.sumsq_part = (float*)(w + L.gssq);
    g.counters = (int*)(w + L.counters);
    timer_begin(timer, stage, s);
    const int r = launch_gemm(g, p, s);
    timer_end(timer, s);
    return r;
  };

  timer_begin(timer, ST_DRAFT_SELECT, s);
  hipLaunchKernelGGL(draft_init_kernel, dim3(B), dim3(256), 0, s, st);
  timer_end(timer, s);
  // padding rows of the attention output are never written by the attention kernels;
  // zero them once so every row the O projection reads is finite
  rc = launch_fill_zero(att, (size_t)B * F * Hq * Dh * 2, s);
  if (rc) return rc;

  for (int level = 1; level <= pr->depth; ++level) {
    const int i = level == 1 ? 0 : 1;
    const int FL = level == 1 ? 1 : F;
    const int Rl = B * FL;
    st.level = level;
    st.FL = FL;
    st.FLprev = level <= 2 ? 1 : F;
    st.h = level == 1 ? nullptr : h;
    st.n_tk = L.p_lm[i].n_tiles;

    timer_begin(timer, ST_DRAFT_SELECT, s);
    hipLaunchKernelGGL(draft_prep_kernel, dim3(B, 1 + st.FLprev), dim3(256), 0, s, st);
    timer_end(timer, s);
    // FC over [parent feature ; token embedding] -> x, bf16(ln_attn * x), row sums of squares
    {
      GemmDesc g{};
      g.w0 = w_fc;
      g.w_layout = lw->layout;
      g.n = H;
      g.k = 2 * H;
      g.ldw = 2 * H;
      g.m = Rl;
      g.x.a = bseg(st.feat, H, st.feat_idx);
      g.x.b = bseg(embed, H, st.tok);
      g.x.ka = H;
      g.epi.kind = EPI_RESID;
      g.epi.out = x;
      g.epi.ld_out = H;
      g.epi.xn_out = x16;
      g.epi.xn_gain = lw->ln_attn;
      g.epi.ssq_out = ssq_x;
      if ((rc = gemm(g, L.p_fc[i], ST_DRAFT_FC))) return rc;
    }
    // RMSNorm -> QKV -> rotary at the node positions; k/v into the nodes' slots
    {
      GemmDesc g{};
      g.w0 = lw->w_qkv;
      g.w_layout = lw->layout;
      g.n = (Hq + 2 * Hkv) * Dh;
      g.k = H;
      g.ldw = H;
      g.m = Rl;
      g.x.a = bseg(x16, H, nullptr);
      g.x.b = g.x.a;
      g.x.ka = H;
      g.x.norm = 2;
      g.x.ssq_in = ssq_x;
      g.x.np = L.p_fc[i].n_tiles;
      g.x.eps = d->rms_eps;
      g.epi.kind = EPI_QKV;
      g.epi.q_out = qb;
      g.epi.k_out = kd;
      g.epi.v_out = vd;
      g.epi.out_dtype = EAGLE_BF16;
      g.epi.pos = st.pos;
      g.epi.kv_idx = st.kv_idx;
      g.epi.hq = Hq;
      g.epi.hkv = Hkv;
      g.epi.hd = Dh;
      g.epi.theta = d->rope_theta;
      if ((rc = gemm(g, L.p_qkv[i], ST_QKV))) return rc;
    }
    // attention of the frontier rows over [draft KV prefix ; expanded nodes on their root path]
    {
      AttnArgs a{};
      a.dtype = EAGLE_BF16;
      a.batch = B;
      a.hq = Hq;
      a.hkv = Hkv;
      a.hd = Dh;
      a.q = qb;
      a.k_cache = dk_cache;
      a.v_cache = dv_cache;
      a.cb = cache->batch_stride;
      a.ch = cache->head_stride;
      a.ct = cache->token_stride;
      a.cap = cache->capacity;
      a.table = cache->block_table;
      a.ps = cache->page_size;
      a.maxb = cache->max_blocks;
      a.npages = cache->n_pages;
      a.k_tree = kd;
      a.v_tree = vd;
      a.anc = st.anc;
      a.mw = 1;
      a.tree_off = st.att_off;
      a.prefix_len = prefix_len;
      a.max_nodes = FL;
      a.max_prefix = max_prefix;
      a.n_nodes = st.cnt + C_NNODES * B;
      a.q_lo = st.cnt + C_QLO * B;
      a.q_stride = FL;
      a.out = att;
      a.part_o = (float*)(w + L.attn_part);
      a.part_ml = a.part_o + (size_t)B * Hkv * L.pa[i].n_chunks * L.pa[i].rmax * Dh;
      if ((rc = launch_attn(a, L.pa[i], timer, s))) return rc;
    }
    // O + residual x -> y; bf16(ln_mlp * y) and row sums of squares
    {
      GemmDesc g{};
      g.w0 = lw->w_o;
      g.w_layout = lw->layout;
      g.n = H;
      g.k = Hq * Dh;
      g.ldw = Hq * Dh;
      g.m = Rl;
      g.x.a = bseg(att, Hq * Dh, nullptr);
      g.x.b = g.x.a;
      g.x.ka = Hq * Dh;
      g.epi.kind = EPI_RESID;
      g.epi.out = y;
      g.epi.ld_out = H;
      g.epi.resid = x;
      g.epi.resid_dtype = EAGLE_F32;
      g.epi.ld_resid = H;
      g.epi.xn_out = y16;
      g.epi.xn_gain = lw->ln_mlp;
      g.epi.ssq_out = ssq_y;
      if ((rc = gemm(g, L.p_o[i], ST_O))) return rc;
    }
    // RMSNorm -> gate/up -> SiLU(gate) * up
    {
      GemmDesc g{};
      g.w0 = lw->w_gate;
      g.w1 = lw->w_up;
      g.w_layout = lw->layout;
      g.dual = 1;
      g.n = Fm;
      g.k = H;
      g.ldw = H;
      g.m = Rl;
      g.x.a = bseg(y16, H, nullptr);
      g.x.b = g.x.a;
      g.x.ka = H;
      g.x.norm = 2;
      g.x.ssq_in = ssq_y;
      g.x.np = L.p_o[i].n_tiles;
      g.x.eps = d->rms_eps;
      g.epi.kind = EPI_SILU;
      g.epi.act = act;
      g.epi.act_dtype = EAGLE_BF16;
      g.epi.ld_act = Fm;
      if ((rc = gemm(g, L.p_gu[i], ST_GATE_UP))) return rc;
    }
    // down + residual y -> f_hat (fp32); bf16(final_ln * f_hat) and row sums of squares
    {
      GemmDesc g{};
      g.w0 = lw->w_down;
      g.w_layout = lw->layout;
      g.n = H;
      g.k = Fm;
      g.ldw = Fm;
      g.m = Rl;
      g.x.a = bseg(act, Fm, nullptr);
      g.x.b = g.x.a;
      g.x.ka = Fm;
      g.epi.kind = EPI_RESID;
      g.epi.out = h;
      g.epi.ld_out = H;
      g.epi.resid = y;
      g.epi.resid_dtype = EAGLE_F32;
      g.epi.ld_resid = H;
      g.epi.xn_out = h16;
      g.epi.xn_gain = final_ln;
      g.epi.ssq_out = ssq_h;
      if ((rc = gemm(g, L.p_down[i], ST_DOWN))) return rc;
    }
    // final RMSNorm -> LM head with per-tile top-k and (max, sum exp)
    {
      GemmDesc g{};
      g.w0 = w_lm;
      g.w_layout = d->lm_layout;
      g.n = V;
      g.k = H;
      g.ldw = H;
      g.m = Rl;
      g.x.a = bseg(h16, H, nullptr);
      g.x.b = g.x.a;
      g.x.ka = H;
      g.x.norm = 2;
      g.x.ssq_in = ssq_h;
      g.x.np = L.p_down[i].n_tiles;
      g.x.eps = d->rms_eps;
      g.epi.kind = EPI_TOPK;
      g.epi.topk_val = (float*)(w + L.tk_val);
      g.epi.topk_idx = (int32_t*)(w + L.tk_idx);
      g.epi.lse_part = (float*)(w + L.tk_lse);
      g.epi.topk = K;
      g.epi.n_part = L.p_lm[i].n_tiles;
      if ((rc = gemm(g, L.p_lm[i], ST_LM_HEAD))) return rc;
    }
    timer_begin(timer, ST_DRAFT_TOPK, s);
    if (pr->top_k <= 10)
      hipLaunchKernelGGL(draft_topk_merge_kernel<10>, dim3(Rl), dim3(256), 0, s, st);
    else if (pr->top_k <= 12)
      hipLaunchKernelGGL(draft_topk_merge_kernel<12>, dim3(Rl), dim3(256), 0, s, st);
    else
      hipLaunchKernelGGL(draft_topk_merge_kernel<16>, dim3(Rl), dim3(256), 0, s, st);
    timer_end(timer, s);
    timer_begin(timer, ST_DRAFT_SELECT, s);
    hipLaunchKernelGGL(draft_select_kernel, dim3(B), dim3(256), 0, s, st);
    timer_end(timer, s);
  }
  timer_begin(timer, ST_DRAFT_SELECT, s);
  hipLaunchKernelGGL(draft_rerank_kernel, dim3(B), dim3(256), 0, s, st, tree_off, parent, tokens, cum_logp);
  timer_end(timer, s);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int draft_pool_impl(const eagle_dims* d, const eagle_draft_params* pr, int B, int max_prefix, const void* ws,
                    size_t ws_bytes, int32_t* pool_n, int32_t* token, int32_t* parent, int32_t* depth, float* cum,
                    float* logp, int32_t* expanded, hipStream_t s) {
  int rc = check_draft(d, pr, B, max_prefix);
  if (rc) return rc;
  if (!ws) return EAGLE_ERR_ARG;
  const DraftLayout L = plan_draft(d, pr, B, max_prefix);
  if (ws_bytes < L.total) return EAGLE_ERR_WORKSPACE;
  DraftState st = make_state(L, d, pr, B, (char*)ws);
  hipLaunchKernelGGL(draft_pool_kernel, dim3(B), dim3(256), 0, s, st, pool_n, token, parent, depth, cum, logp,
                     expanded);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle

extern "C" int eagle_draft_expand(const eagle_dims* dims, const eagle_draft_params* params, const void* w_fc,
                                  const eagle_layer_w* draft_layer, const void* final_ln, const void* w_lm,
                                  const void* embed, int32_t batch, const float* root_feature,
                                  const int32_t* root_token, const void* dk_cache, const void* dv_cache,
                                  const eagle_cache_layout* cache, const int32_t* prefix_len, int32_t max_prefix,
                                  int32_t* tree_off, int32_t* parent, int32_t* tokens, float* cum_logp,
                                  void* workspace, size_t ws_bytes, eagle_timer* timer, void* stream) {
  return eagle::draft_expand_impl(dims, params, w_fc, draft_layer, final_ln, w_lm, embed, batch, root_feature,
                                  root_token, dk_cache, dv_cache, cache, prefix_len, max_prefix, tree_off, parent,
                                  tokens, cum_logp, workspace, ws_bytes, timer, (hipStream_t)stream);
}

extern "C" int eagle_draft_pool(const eagle_dims* dims, const eagle_draft_params* params, int32_t batch,
                                int32_t max_prefix, const void* workspace, size_t ws_bytes, int32_t* pool_n,
                                int32_t* token, int32_t* parent, int32_t* depth, float* cum_logp, float* logp,
                                int32_t* expanded, void* stream) {
  return eagle::draft_pool_impl(dims, params, batch, max_prefix, workspace, ws_bytes, pool_n, token, parent, depth,
                                cum_logp, logp, expanded, (hipStream_t)stream);
}
