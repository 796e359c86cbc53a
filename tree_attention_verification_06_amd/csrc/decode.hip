// Draft KV update after acceptance (gfx950): the draft head's cache slots of the committed
// path, recomputed from the target's true features.
//
// "Speculative decoding with EAGLE", Technical insight: the draft works on the target's
// hidden features and is fed the true embedding of the next token.  During expansion the
// draft rows of deeper nodes use the draft's own predicted features; once the target has
// verified the tree, the committed positions P .. P + L get the rows the draft would have
// seen with the target's features:
//   slot P + d  <-  K/V of the draft layer for W_fc [f ; E[token of path node d]] at
//                  position P + d, f = the step's root feature (d = 0) or the target
//                  feature h of path node d - 1 (d >= 1).
// Only the draft layer's K and V are needed (RMSNorm -> K/V rows of W_qkv -> rotary on K),
// so the update is the draft's FC and QKV GEMMs over B * (max_accept + 1) rows (rows past
// a sequence's accepted length are inert: their K/V are dropped) plus a gather and a scatter.
#include <algorithm>

#include "gemm.h"

namespace eagle {

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DkvLayout {
  GemmPlan p_fc, p_qkv;
  size_t stage, rows, x, x16, ssq, q, k, v, gpart, gssq, counters, total;
};

DkvLayout plan_dkv(const eagle_dims* d, int B, int S) {
  DkvLayout L{};
  const int R = B * S;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  L.p_fc = plan_gemm(EAGLE_BF16, H, 2 * H, R, 0, EPI_RESID, D);
  L.p_qkv = plan_gemm(EAGLE_BF16, (Hq + 2 * Hkv) * D, H, R, 0, EPI_QKV, D);
  size_t pf = 0, sf = 0, ci = 0;
  for (const GemmPlan* p : {&L.p_fc, &L.p_qkv}) {
    size_t a, b, c;
    gemm_workspace(*p, &a, &b, &c);
    pf = std::max(pf, a);
    sf = std::max(sf, b);
    ci = std::max(ci, c);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(std::max<size_t>(bytes, 1));
    return o;
  };
  L.stage = take((size_t)R * H * 2);
  L.rows = take((size_t)R * 4 * 4);  // tok | pos | kv row | cache slot
  L.x = take((size_t)R * H * 4);
  L.x16 = take((size_t)R * H * 2);
  L.ssq = take((size_t)std::max(L.p_fc.n_tiles, 1) * R * 4);
  L.q = take((size_t)R * Hq * D * 2);
  L.k = take((size_t)R * Hkv * D * 2);
  L.v = take((size_t)R * Hkv * D * 2);
  L.gpart = take(pf * 4);
  L.gssq = take(sf * 4);
  L.counters = take(ci * 4);
  L.total = off;
  return L;
}

struct DkvArgs {
  int S, H, hkv, hd;
  const int32_t* tree_off;
  const int32_t* tokens;
  const int32_t* accept_len;
  const int32_t* path;
  const int32_t* prefix_len;
  const float* h_nodes;
  const float* root_feature;
  bf16* stage;
  int32_t *tok, *pos, *kvi, *cslot;
  const bf16* k;
  const bf16* v;
  bf16* dk_cache;
  bf16* dv_cache;
  CacheView cv;
  int cap;
  int32_t* status;
};

__device__ __forceinline__ void set_status(int32_t* st, int code) {
  if (st) atomicCAS(st, 0, code);
}

// Workgroup (b, d): row r = b * S + d.  Active iff accept_len[b] >= 0 and d <= accept_len[b]:
// the bf16 feature row (root feature, or h of path node d - 1), the token of path node d,
// position and cache slot P + d with P = prefix_len[b] - L - 1 (prefix_len already
// advanced by the commit).  Inactive rows read the root feature and token 0 and are dropped.
__global__ __launch_bounds__(256) void draft_kv_prep_kernel(DkvArgs a) {
  const int b = blockIdx.x, d = blockIdx.y, r = b * a.S + d;
  const int L = a.accept_len[b];
  const bool active = L >= 0 && d <= L;
  const int off = a.tree_off[b];
  const float* src = a.root_feature + (int64_t)b * a.H;
  if (active && d > 0) src = a.h_nodes + (int64_t)(off + a.path[(int64_t)b * a.S + d - 1]) * a.H;
  for (int c = threadIdx.x * 4; c < a.H; c += blockDim.x * 4) {
    const float4 v = *(const float4*)(src + c);
    *(uint2*)(a.stage + (int64_t)r * a.H + c) = make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
  }
  if (threadIdx.x == 0) {
    const int P = active ? a.prefix_len[b] - L - 1 : 0;
    a.tok[r] = active ? a.tokens[off + a.path[(int64_t)b * a.S + d]] : 0;
    a.pos[r] = active ? P + d : 0;
    a.kvi[r] = active ? r : -1;
    a.cslot[r] = active ? P + d : -1;
  }
}

// Workgroup (b, d): the K and V rows of row r into the draft cache slot cslot[r] of
// sequence b (16-byte copies), or nothing for an inactive row.
__global__ __launch_bounds__(256) void draft_kv_scatter_kernel(DkvArgs a) {
  const int b = blockIdx.x, r = b * a.S + blockIdx.y;
  const int slot = a.cslot[r];
  if (slot < 0) return;
  if (slot >= a.cap) {
    if (threadIdx.x == 0) set_status(a.status, EAGLE_ERR_CAPACITY);
    return;
  }
  bool ok;
  const int64_t row0 = cache_offset(a.cv, b, 0, slot, ok);  // the slot's offset at head 0
  if (!ok) {
    if (threadIdx.x == 0) set_status(a.status, EAGLE_ERR_ARG);
    return;
  }
  const int chunks = a.hd / 8;
  const int per = a.hkv * chunks;
  for (int i = threadIdx.x; i < 2 * per; i += blockDim.x) {
    const int which = i / per, j = i % per, h = j / chunks, c = j % chunks;
    const uint4 v = *(const uint4*)((which ? a.v : a.k) + ((int64_t)r * a.hkv + h) * a.hd + c * 8);
    *(uint4*)((which ? a.dv_cache : a.dk_cache) + row0 + (int64_t)h * a.cv.ch + c * 8) = v;
  }
}

int check_dkv(const eagle_dims* d, int B, int max_accept) {
  if (!d || B < 1 || max_accept < 0 || max_accept > 127) return EAGLE_ERR_ARG;
  if (d->dtype != EAGLE_BF16 || d->head_dim != 128 || d->rms_eps <= 0.f || d->hidden <= 0 || d->hidden % 64 ||
      d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads || d->vocab < 1)
    return EAGLE_ERR_UNSUPPORTED;
  return EAGLE_OK;
}

}  // namespace

size_t draft_kv_workspace(const eagle_dims* d, int B, int max_accept) {
  if (check_dkv(d, B, max_accept)) return 0;
  return plan_dkv(d, B, max_accept + 1).total;
}

int draft_kv_commit_impl(const eagle_dims* d, const void* w_fc, const eagle_layer_w* lw, const void* embed, int B,
                         const int32_t* tree_off, const int32_t* tokens, const float* h_nodes,
                         const float* root_feature, const int32_t* accept_len, const int32_t* path, int max_accept,
                         const int32_t* prefix_len, void* dk_cache, void* dv_cache, const eagle_cache_layout* cache,
                         int32_t* dev_status, void* ws, size_t ws_bytes, hipStream_t s) {
  int rc = check_dkv(d, B, max_accept);
  if (rc) return rc;
  if (!w_fc || !lw || !lw->ln_attn || !lw->w_qkv || !embed || !tree_off || !tokens || !h_nodes || !root_feature ||
      !accept_len || !path || !prefix_len || !dk_cache || !dv_cache || !cache || !ws)
    return EAGLE_ERR_ARG;
  if (lw->layout != 0 && lw->layout != 1) return EAGLE_ERR_ARG;
  if (((uintptr_t)ws) & 255) return EAGLE_ERR_ARG;
  if (check_cache_layout(cache)) return EAGLE_ERR_ARG;
  const int S = max_accept + 1, R = B * S;
  const DkvLayout L = plan_dkv(d, B, S);
  if (ws_bytes < L.total) return EAGLE_ERR_WORKSPACE;
  char* w = (char*)ws;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  DkvArgs a{};
  a.S = S;
  a.H = H;
  a.hkv = Hkv;
  a.hd = D;
  a.tree_off = tree_off;
  a.tokens = tokens;
  a.accept_len = accept_len;
  a.path = path;
  a.prefix_len = prefix_len;
  a.h_nodes = h_nodes;
  a.root_feature = root_feature;
  a.stage = (bf16*)(w + L.stage);
  int32_t* rows = (int32_t*)(w + L.rows);
  a.tok = rows;
  a.pos = rows + R;
  a.kvi = rows + 2 * R;
  a.cslot = rows + 3 * R;
  a.k = (const bf16*)(w + L.k);
  a.v = (const bf16*)(w + L.v);
  a.dk_cache = (bf16*)dk_cache;
  a.dv_cache = (bf16*)dv_cache;
  a.cv = cache_view(cache);
  a.cap = cache->capacity;
  a.status = dev_status;
  float* ssq = (float*)(w + L.ssq);
  void* x16 = w + L.x16;
  auto gemm = [&](GemmDesc& g, const GemmPlan& p) {
    g.dtype = EAGLE_BF16;
    g.partials = (float*)(w + L.gpart);
    g.sumsq_part = (float*)(w + L.gssq);
    g.counters = (int*)(w + L.counters);
    return launch_gemm(g, p, s);
  };
  auto bseg = [](const void* p, int64_t ld, const int32_t* idx) {
    XSeg sg;
    sg.ptr = p;
    sg.dtype = EAGLE_BF16;
    sg.ld = ld;
    sg.idx = idx;
    return sg;
  };

  hipLaunchKernelGGL(draft_kv_prep_kernel, dim3(B, S), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return EAGLE_ERR_HIP;
  // FC over [feature ; token embedding] -> x, bf16(ln_attn * x), row sums of squares
  {
    GemmDesc g{};
    g.w0 = w_fc;
    g.w_layout = lw->layout;
    g.n = H;
    g.k = 2 * H;
    g.ldw = 2 * H;
    g.m = R;
    g.x.a = bseg(a.stage, H, nullptr);
    g.x.b = bseg(embed, H, a.tok);
    g.x.ka = H;
    g.epi.kind = EPI_RESID;
    g.epi.out = (float*)(w + L.x);
    g.epi.ld_out = H;
    g.epi.xn_out = x16;
    g.epi.xn_gain = lw->ln_attn;
    g.epi.ssq_out = ssq;
    if ((rc = gemm(g, L.p_fc))) return rc;
  }
  // RMSNorm -> QKV -> rotary at the positions; K/V of active rows into rows kvi (q unused)
  {
    GemmDesc g{};
    g.w0 = lw->w_qkv;
    g.w_layout = lw->layout;
    g.n = (Hq + 2 * Hkv) * D;
    g.k = H;
    g.ldw = H;
    g.m = R;
    g.x.a = bseg(x16, H, nullptr);
    g.x.b = g.x.a;
    g.x.ka = H;
    g.x.norm = 2;
    g.x.ssq_in = ssq;
    g.x.np = L.p_fc.n_tiles;
    g.x.eps = d->rms_eps;
    g.epi.kind = EPI_QKV;
    g.epi.q_out = w + L.q;
    g.epi.k_out = w + L.k;
    g.epi.v_out = w + L.v;
    g.epi.out_dtype = EAGLE_BF16;
    g.epi.pos = a.pos;
    g.epi.kv_idx = a.kvi;
    g.epi.hq = Hq;
    g.epi.hkv = Hkv;
    g.epi.hd = D;
    g.epi.theta = d->rope_theta;
    if ((rc = gemm(g, L.p_qkv))) return rc;
  }
  hipLaunchKernelGGL(draft_kv_scatter_kernel, dim3(B, S), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle

extern "C" int eagle_draft_kv_commit(const eagle_dims* dims, const void* w_fc, const eagle_layer_w* draft_layer,
                                     const void* embed, int32_t batch, const int32_t* tree_off, const int32_t* tokens,
                                     const float* h_nodes, const float* root_feature, const int32_t* accept_len,
                                     const int32_t* path, int32_t max_accept, const int32_t* prefix_len,
                                     void* dk_cache, void* dv_cache, const eagle_cache_layout* cache,
                                     int32_t* dev_status, void* workspace, size_t ws_bytes, void* stream) {
  return eagle::draft_kv_commit_impl(dims, w_fc, draft_layer, embed, batch, tree_off, tokens, h_nodes, root_feature,
                                     accept_len, path, max_accept, prefix_len, dk_cache, dv_cache, cache, dev_status,
                                     workspace, ws_bytes, (hipStream_t)stream);
}
