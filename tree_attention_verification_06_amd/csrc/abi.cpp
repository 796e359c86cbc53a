// C entry points: argument checks, workspace layout and the launch sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "attn.h"
#include "common.h"
#include "draft.h"
#include "gemm.h"
#include "tree.h"

struct eagle_timer {
  int cap = 0;
  int n = 0;
  bool open = false;
  uint32_t mask = 0xffffffffu;
  std::vector<hipEvent_t> ev;
  std::vector<int> stage;
};

namespace eagle {

// A stage whose event cannot be recorded is left out of the timer (its slot is reused).
void timer_begin(eagle_timer* t, int stage, hipStream_t s) {
  if (!t || t->n >= t->cap || !((t->mask >> stage) & 1u)) return;
  if (hipEventRecord(t->ev[2 * t->n], s) != hipSuccess) return;
  t->stage[t->n] = stage;
  t->open = true;
}
void timer_end(eagle_timer* t, hipStream_t s) {
  if (!t || !t->open) return;
  t->open = false;
  if (hipEventRecord(t->ev[2 * t->n + 1], s) != hipSuccess) return;
  t->n++;
}

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int elem_size(int dtype) { return dtype == EAGLE_BF16 ? 2 : 4; }

int check_dims(const eagle_dims* d) {
  if (!d) return EAGLE_ERR_ARG;
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->vocab <= 0 || d->ffn < 0)
    return EAGLE_ERR_ARG;
  if (d->n_q_heads % d->n_kv_heads) return EAGLE_ERR_UNSUPPORTED;
  if (d->hidden % 64 || d->ffn % 64) return EAGLE_ERR_UNSUPPORTED;
  if (d->dtype == EAGLE_BF16) {
    if (d->head_dim != 128) return EAGLE_ERR_UNSUPPORTED;
  } else if (d->dtype == EAGLE_F32) {
    if (d->head_dim != 64 && d->head_dim != 128) return EAGLE_ERR_UNSUPPORTED;
  } else {
    return EAGLE_ERR_UNSUPPORTED;
  }
  if ((d->ffn == 0) != (d->rms_eps == 0.f)) return EAGLE_ERR_UNSUPPORTED;
  if (d->rms_eps < 0.f || d->rope_theta < 0.f) return EAGLE_ERR_ARG;
  if (d->lm_layout != 0 && d->lm_layout != 1) return EAGLE_ERR_ARG;
  if (d->lm_layout == 1 && d->dtype != EAGLE_BF16) return EAGLE_ERR_UNSUPPORTED;
  return EAGLE_OK;
}

struct VerifyLayout {
  size_t q, attn, y, act, attn_part, gemm_part, gemm_ssq, counters, keys, done, total;
  size_t gparent, row_tree, samp_part;  // sampling LM head only
  size_t y16, h16, ssq_y, ssq_h;  // bf16 path: gain-scaled bf16 copies and row sum-of-squares partials
  GemmPlan p_qkv, p_o, p_gu, p_down, p_lm;
  AttnPlan pa;
};

VerifyLayout plan_verify(const eagle_dims* d, int B, int total_nodes, int max_nodes, int max_prefix,
                         bool sample = false) {
  VerifyLayout L{};
  const int es = elem_size(d->dtype);
  const int M = total_nodes;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim, F = d->ffn, V = d->vocab;
  L.p_qkv = plan_gemm(d->dtype, (Hq + 2 * Hkv) * D, H, M, 0, EPI_QKV, D);
  L.p_o = plan_gemm(d->dtype, H, Hq * D, M, 0, EPI_RESID, D);
  if (F > 0) {
    L.p_gu = plan_gemm(d->dtype, F, H, M, 1, EPI_SILU, D);
    L.p_down = plan_gemm(d->dtype, H, F, M, 0, EPI_RESID, D);
  }
  L.p_lm = plan_gemm(d->dtype, V, H, M, 0, sample ? EPI_SAMPLE : EPI_ARGMAX, D);
  L.pa = plan_attn(d->dtype, B, Hq, Hkv, D, max_nodes, max_prefix);
  size_t pf = 0, sf = 0, ci = 0;
  for (const GemmPlan* p : {&L.p_qkv, &L.p_o, &L.p_gu, &L.p_down, &L.p_lm}) {
    if (p->n_tiles == 0) continue;
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
  L.q = take((size_t)M * Hq * D * es);
  L.attn = take((size_t)M * Hq * D * es);
  L.y = take((size_t)M * H * 4);
  L.act = take((size_t)M * std::max(F, 1) * es);
  L.attn_part = take(attn_workspace_floats(L.pa, B, Hkv, D) * 4);
  L.gemm_part = take(pf * 4);
  L.gemm_ssq = take(sf * 4);
  L.counters = take(ci * 4);
  L.keys = take((size_t)M * 8);
  L.done = take(4);
  L.y16 = take((size_t)M * H * 2);
  L.h16 = take((size_t)M * H * 2);
  L.ssq_y = take((size_t)std::max(L.p_o.n_tiles, 1) * M * 4);
  L.ssq_h = take((size_t)std::max(F > 0 ? L.p_down.n_tiles : L.p_o.n_tiles, 1) * M * 4);
  if (sample) {
    L.gparent = take((size_t)M * 4);
    L.row_tree = take((size_t)M * 4);
    L.samp_part = take((size_t)M * L.p_lm.n_tiles * 16);
  }
  L.total = off;
  return L;
}

GemmDesc base_desc(const eagle_dims* d) {
  GemmDesc g{};
  g.dtype = d->dtype;
  return g;
}

XSeg seg(const void* p, int dtype, int64_t ld, const int32_t* idx = nullptr) {
  XSeg s;
  s.ptr = p;
  s.dtype = dtype;
  s.ld = ld;
  s.idx = idx;
  return s;
}

// Workspace of eagle_fuse_features: the split-K partials, sums of squares and counters of
// its one GEMM (H outputs over K = 3H for `batch` rows).
struct FuseLayout {
  GemmPlan plan;
  size_t part, ssq, counters, total;
};
FuseLayout fuse_layout(const eagle_dims* d, int B) {
  FuseLayout L{};
  if (!d || d->dtype != EAGLE_BF16 || B < 1 || d->hidden <= 0 || d->hidden % 64) return L;
  L.plan = plan_gemm(EAGLE_BF16, d->hidden, 3 * d->hidden, B, 0, EPI_STORE_F32, d->head_dim);
  size_t pf, sf, ci;
  gemm_workspace(L.plan, &pf, &sf, &ci);
  size_t off = 0;
  L.part = off;
  off += align256(std::max<size_t>(pf * 4, 1));
  L.ssq = off;
  off += align256(std::max<size_t>(sf * 4, 1));
  L.counters = off;
  off += align256(std::max<size_t>(ci * 4, 1));
  L.total = off;
  return L;
}

}  // namespace

// Outputs of verification at temperature T > 0 (eagle_tree_verify_sample).
struct SampleOut {
  const int32_t* parent;
  float temperature;
  const float* gumbel;
  float* child_logit;
  float* rest_lse;
  int32_t* rest_token;
};

// Verification of every node of every tree: n_layers decoder layers (layers[0..n_layers-1],
// applied in order; layer l reads the caches at l * cache_ls elements and writes its tree
// K/V at l * total_nodes * Hkv * D) + LM head with a fused argmax, or (so != nullptr) with
// the sampling epilogue and its per-row merge.
int verify_impl(const eagle_dims* d, const eagle_layer_w* layers, int n_layers, int64_t cache_ls,
                const void* final_ln, const void* w_lm, int B,
                const int32_t* tree_off, int total_nodes, int max_nodes, const void* x_in, const void* embed,
                const int32_t* tokens, const uint64_t* anc, int mw, const int32_t* pos, const int32_t* prefix_len,
                int max_prefix, const void* k_cache, const void* v_cache, const eagle_cache_layout* cache,
                void* k_tree, void* v_tree, float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn,
                float* dbg_logits, void* ws, size_t ws_bytes, eagle_timer* timer, hipStream_t s,
                const SampleOut* so = nullptr, int (*scratch_of)(void**) = nullptr) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!layers || !w_lm || !tree_off || !anc || !pos || !prefix_len || !k_cache || !v_cache || !cache || !k_tree ||
      !v_tree || !h_out || (!ws && !scratch_of))
    return EAGLE_ERR_ARG;
  if (n_layers < 1 || n_layers > 1024) return EAGLE_ERR_ARG;
  // a stack needs the pre-norm layer with an MLP: the residual stream of layer l > 0 is the
  // previous layer's f32 output, and the down epilogue prepares the next layer's norm
  if (n_layers > 1 && (d->ffn <= 0 || !(d->rms_eps > 0.f))) return EAGLE_ERR_UNSUPPORTED;
  if (n_layers > 1 && cache_ls < 0) return EAGLE_ERR_ARG;
  if (!so && !argmax) return EAGLE_ERR_ARG;
  if (so) {
    if (!so->parent || !tokens || !so->gumbel || !so->child_logit || !so->rest_lse || !so->rest_token)
      return EAGLE_ERR_ARG;
    if (!(so->temperature > 0.f) || !std::isfinite(1.f / so->temperature)) return EAGLE_ERR_ARG;
  }
  if (B < 1 || total_nodes < 1 || max_nodes < 1 || max_nodes > 64 * mw || mw < 1 || mw > 2 || max_prefix < 0)
    return EAGLE_ERR_ARG;
  if (!x_in && (!embed || !tokens)) return EAGLE_ERR_ARG;
  const bool norm = d->rms_eps > 0.f;
  if (norm && !final_ln) return EAGLE_ERR_ARG;
  for (int l = 0; l < n_layers; ++l) {
    const eagle_layer_w* lw = layers + l;
    if (!lw->w_qkv || !lw->w_o) return EAGLE_ERR_ARG;
    if (lw->layout != 0 && lw->layout != 1) return EAGLE_ERR_ARG;
    if (lw->layout == 1 && d->dtype != EAGLE_BF16) return EAGLE_ERR_UNSUPPORTED;
    if (norm && (!lw->ln_attn || !lw->ln_mlp || !lw->w_gate || !lw->w_up || !lw->w_down)) return EAGLE_ERR_ARG;
  }
  if (((uintptr_t)ws) & 255) return EAGLE_ERR_ARG;
  if (check_cache_layout(cache)) return EAGLE_ERR_ARG;
  const VerifyLayout L = plan_verify(d, B, total_nodes, max_nodes, max_prefix, so != nullptr);
  if (ws_bytes < L.total) return EAGLE_ERR_WORKSPACE;
  if (scratch_of) {  // the library's own buffer, resolved once every argument has passed
    rc = scratch_of(&ws);
    if (rc) return rc;
  }
  char* w = (char*)ws;
  const int dt = d->dtype;
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim, F = d->ffn, V = d->vocab;
  const int M = total_nodes;
  void* q = w + L.q;
  void* attn = w + L.attn;
  float* y = (float*)(w + L.y);
  void* act = w + L.act;
  float* gpart = (float*)(w + L.gemm_part);
  float* gssq = (float*)(w + L.gemm_ssq);
  int* counters = (int*)(w + L.counters);
  unsigned long long* keys = (unsigned long long*)(w + L.keys);
  int* done = (int*)(w + L.done);

  // x: the given node states, or the token embeddings
  const XSeg xseg = x_in ? seg(x_in, dt, H) : seg(embed, dt, H, tokens);
  const bool bf = dt == EAGLE_BF16;
  void* y16 = w + L.y16;
  void* h16 = w + L.h16;
  float* ssq_y = (float*)(w + L.ssq_y);
  float* ssq_h = (float*)(w + L.ssq_h);
  auto common = [&](GemmDesc& g) {
    g.partials = gpart;
    g.sumsq_part = gssq;
    g.counters = counters;
  };

  if (scratch_of) {
    // the split-K counters, argmax keys and completion counter must start at zero; every
    // call leaves them so, but a shared buffer is cleared anyway (a fill kernel, so the
    // call can be captured into a graph)
    rc = launch_fill_zero(w + L.counters, L.done + 4 - L.counters, s);
    if (rc) return rc;
  }
  int32_t* gparent = so ? (int32_t*)(w + L.gparent) : nullptr;
  int32_t* row_tree = so ? (int32_t*)(w + L.row_tree) : nullptr;
  float4* samp_part = so ? (float4*)(w + L.samp_part) : nullptr;
  if (so) {
    // 0. each row's global parent row and sequence, for the sampling LM head
    timer_begin(timer, ST_OTHER, s);
    rc = launch_sample_prep(tree_off, so->parent, B, M, gparent, row_tree, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  const int64_t tree_ls = (int64_t)M * Hkv * D;  // elements between two layers' tree K/V
  for (int l = 0; l < n_layers; ++l) {
  const eagle_layer_w* lw = layers + l;
  const bool first = l == 0;
  const eagle_layer_w* next = l + 1 < n_layers ? layers + l + 1 : nullptr;
  void* k_tree_l = (char*)k_tree + (size_t)l * tree_ls * elem_size(dt);
  void* v_tree_l = (char*)v_tree + (size_t)l * tree_ls * elem_size(dt);
  // 1. RMSNorm -> QKV projection -> rotary at pos -> q (workspace), k_tree, v_tree.  Layer
  //    l > 0 reads the previous layer's output: on the bf16 path as bf16(ln_attn * h) and
  //    row sums of squares written by that layer's down epilogue
  {
    GemmDesc g = base_desc(d);
    g.w0 = lw->w_qkv;
    g.w_layout = lw->layout;
    g.n = (Hq + 2 * Hkv) * D;
    g.k = H;
    g.ldw = H;
    g.m = M;
    if (first) {
      g.x.a = xseg;
      g.x.norm = norm ? 1 : 0;
      g.x.gain = norm ? lw->ln_attn : nullptr;
    } else if (bf) {
      g.x.a = seg(h16, dt, H);
      g.x.norm = 2;
      g.x.ssq_in = ssq_h;
      g.x.np = L.p_down.n_tiles;
    } else {
      g.x.a = seg(h_out, EAGLE_F32, H);
      g.x.norm = 1;
      g.x.gain = lw->ln_attn;
    }
    g.x.b = g.x.a;
    g.x.ka = H;
    g.x.gain_dtype = dt;
    g.x.eps = d->rms_eps;
    g.epi.kind = EPI_QKV;
    g.epi.q_out = q;
    g.epi.k_out = k_tree_l;
    g.epi.v_out = v_tree_l;
    g.epi.out_dtype = dt;
    g.epi.pos = pos;
    g.epi.hq = Hq;
    g.epi.hkv = Hkv;
    g.epi.hd = D;
    g.epi.theta = d->rope_theta;
    common(g);
    timer_begin(timer, ST_QKV, s);
    rc = launch_gemm(g, L.p_qkv, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  // 2. tree-masked attention -> attn (workspace)
  {
    AttnArgs a{};
    a.dtype = dt;
    a.batch = B;
    a.hq = Hq;
    a.hkv = Hkv;
    a.hd = D;
    a.q = q;
    a.k_cache = (const char*)k_cache + (size_t)l * cache_ls * elem_size(dt);
    a.v_cache = (const char*)v_cache + (size_t)l * cache_ls * elem_size(dt);
    a.cb = cache->batch_stride;
    a.ch = cache->head_stride;
    a.ct = cache->token_stride;
    a.cap = cache->capacity;
    a.table = cache->block_table;
    a.ps = cache->page_size;
    a.maxb = cache->max_blocks;
    a.npages = cache->n_pages;
    a.k_tree = k_tree_l;
    a.v_tree = v_tree_l;
    a.anc = anc;
    a.mw = mw;
    a.tree_off = tree_off;
    a.prefix_len = prefix_len;
    a.max_nodes = max_nodes;
    a.max_prefix = max_prefix;
    a.out = attn;
    a.dbg = l + 1 == n_layers ? dbg_attn : nullptr;
    a.part_o = (float*)(w + L.attn_part);
    a.part_ml = a.part_o + (size_t)B * Hkv * L.pa.n_chunks * L.pa.rmax * D;
    rc = dt == EAGLE_F32 ? launch_attn_f32(a, M, timer, s) : launch_attn(a, L.pa, timer, s);
    if (rc) return rc;
  }
  // 3. O projection + residual -> y (or h_out for the attention-only layer); on the bf16
  //    path the epilogue also writes bf16(gain * y) and row sums of squares for the
  //    next RMSNorm, so the next GEMM streams bf16 activations.  The residual is the
  //    layer input: x (or the token embeddings) for layer 0, h_out (f32) after that
  float* yout = F > 0 ? y : h_out;
  {
    GemmDesc g = base_desc(d);
    g.w0 = lw->w_o;
    g.w_layout = lw->layout;
    g.n = H;
    g.k = Hq * D;
    g.ldw = Hq * D;
    g.m = M;
    g.x.a = seg(attn, dt, Hq * D);
    g.x.b = g.x.a;
    g.x.ka = Hq * D;
    g.epi.kind = EPI_RESID;
    g.epi.out = yout;
    g.epi.ld_out = H;
    if (first) {
      g.epi.resid = x_in ? x_in : embed;
      g.epi.resid_idx = x_in ? nullptr : tokens;
      g.epi.resid_dtype = dt;
    } else {
      g.epi.resid = h_out;
      g.epi.resid_dtype = EAGLE_F32;
    }
    g.epi.ld_resid = H;
    if (bf) {
      g.epi.xn_out = F > 0 ? y16 : h16;
      g.epi.xn_gain = F > 0 ? lw->ln_mlp : final_ln;
      g.epi.ssq_out = F > 0 ? ssq_y : ssq_h;
    }
    common(g);
    timer_begin(timer, ST_O, s);
    rc = launch_gemm(g, L.p_o, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  if (F > 0) {
    // 4. RMSNorm -> gate/up -> SiLU(gate) * up -> act (workspace)
    GemmDesc g = base_desc(d);
    g.w0 = lw->w_gate;
    g.w1 = lw->w_up;
    g.w_layout = lw->layout;
    g.dual = 1;
    g.n = F;
    g.k = H;
    g.ldw = H;
    g.m = M;
    if (bf) {
      g.x.a = seg(y16, dt, H);
      g.x.norm = 2;
      g.x.ssq_in = ssq_y;
      g.x.np = L.p_o.n_tiles;
    } else {
      g.x.a = seg(y, EAGLE_F32, H);
      g.x.norm = 1;
      g.x.gain = lw->ln_mlp;
      g.x.gain_dtype = dt;
    }
    g.x.b = g.x.a;
    g.x.ka = H;
    g.x.eps = d->rms_eps;
    g.epi.kind = EPI_SILU;
    g.epi.act = act;
    g.epi.act_dtype = dt;
    g.epi.ld_act = F;
    common(g);
    timer_begin(timer, ST_GATE_UP, s);
    rc = launch_gemm(g, L.p_gu, s);
    timer_end(timer, s);
    if (rc) return rc;
    // 5. down projection + residual -> h_out (and bf16(gain * h) + row sums of squares,
    //    with the next layer's attention gain, or the final gain after the last layer)
    GemmDesc g2 = base_desc(d);
    g2.w0 = lw->w_down;
    g2.w_layout = lw->layout;
    g2.n = H;
    g2.k = F;
    g2.ldw = F;
    g2.m = M;
    g2.x.a = seg(act, dt, F);
    g2.x.b = g2.x.a;
    g2.x.ka = F;
    g2.epi.kind = EPI_RESID;
    g2.epi.out = h_out;
    g2.epi.ld_out = H;
    g2.epi.resid = y;
    g2.epi.resid_dtype = EAGLE_F32;
    g2.epi.ld_resid = H;
    if (bf) {
      g2.epi.xn_out = h16;
      g2.epi.xn_gain = next ? next->ln_attn : final_ln;
      g2.epi.ssq_out = ssq_h;
    }
    common(g2);
    timer_begin(timer, ST_DOWN, s);
    rc = launch_gemm(g2, L.p_down, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  }  // layers
  // 6. final RMSNorm -> LM head with fused row argmax
  {
    GemmDesc g = base_desc(d);
    g.w0 = w_lm;
    g.w_layout = d->lm_layout;
    g.n = V;
    g.k = H;
    g.ldw = H;
    g.m = M;
    if (bf) {
      g.x.a = seg(h16, dt, H);
      g.x.norm = norm ? 2 : 0;
      g.x.ssq_in = ssq_h;
      g.x.np = F > 0 ? L.p_down.n_tiles : L.p_o.n_tiles;
    } else {
      g.x.a = seg(h_out, EAGLE_F32, H);
      g.x.norm = norm ? 1 : 0;
      g.x.gain = norm ? final_ln : nullptr;
      g.x.gain_dtype = dt;
    }
    g.x.b = g.x.a;
    g.x.ka = H;
    g.x.eps = d->rms_eps;
    if (so) {
      g.epi.kind = EPI_SAMPLE;
      g.epi.noise = so->gumbel;
      g.epi.ld_noise = V;
      g.epi.row_group = row_tree;
      g.epi.inv_t = 1.f / so->temperature;
      g.epi.gparent = gparent;
      g.epi.ctoken = tokens;
      g.epi.max_nodes = max_nodes;
      g.epi.child_logit = so->child_logit;
      g.epi.samp_part = samp_part;
      g.epi.n_part = L.p_lm.n_tiles;
    } else {
      g.epi.kind = EPI_ARGMAX;
      g.epi.keys = keys;
      g.epi.dbg_logits = dbg_logits;
      g.epi.ld_logits = V;
      g.epi.argmax_out = argmax;
      g.epi.max_out = maxlogit;
      g.epi.done = done;
    }
    common(g);
    timer_begin(timer, ST_LM_HEAD, s);
    rc = launch_gemm(g, L.p_lm, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  if (so) {
    // 7. per row: log-normaliser and best noisy token of the non-child tokens
    timer_begin(timer, ST_OTHER, s);
    rc = launch_sample_merge(samp_part, L.p_lm.n_tiles, M, so->rest_lse, so->rest_token, s);
    timer_end(timer, s);
    if (rc) return rc;
  }
  return EAGLE_OK;
}

size_t verify_workspace(const eagle_dims* d, int B, int total_nodes, int max_nodes, int max_prefix,
                        bool sample = false) {
  if (check_dims(d) || B < 1 || total_nodes < 1 || max_nodes < 1) return 0;
  return plan_verify(d, B, total_nodes, max_nodes, max_prefix, sample).total;
}

// Checks the arguments both acceptance rules share and fills the commit half of a.
int commit_args(AcceptArgs& a, int batch, const int32_t* tree_off, int max_nodes, const int32_t* parent,
                const int32_t* tokens, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                const eagle_cache_layout* cache, int n_kv_heads, int head_dim, int dtype, int32_t* prefix_len,
                const float* h_nodes, int hidden, float* next_feature, int max_accept, int32_t* accept_len,
                int32_t* path, int32_t* out_tokens, int32_t* next_token, int32_t* dev_status) {
  if (batch < 1 || max_nodes < 1 || !tree_off || !parent || !tokens || !k_tree || !v_tree || !k_cache || !v_cache ||
      !cache || !prefix_len || !accept_len || !path || !out_tokens || !next_token)
    return EAGLE_ERR_ARG;
  if (max_accept < 0 || max_accept > 127) return EAGLE_ERR_ARG;
  if (dtype != EAGLE_BF16 && dtype != EAGLE_F32) return EAGLE_ERR_UNSUPPORTED;
  const int es = elem_size(dtype);
  if (n_kv_heads < 1 || head_dim < 1 || (head_dim * es) % 16) return EAGLE_ERR_UNSUPPORTED;
  if ((cache->token_stride * es) % 16 || (cache->head_stride * es) % 16 || (cache->batch_stride * es) % 16)
    return EAGLE_ERR_ARG;
  if (cache->block_table && check_cache_layout(cache)) return EAGLE_ERR_ARG;  // the paging fields
  if (next_feature && (!h_nodes || hidden < 1 || hidden % 4)) return EAGLE_ERR_ARG;
  a.tree_off = tree_off;
  a.parent = parent;
  a.tokens = tokens;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.capacity = cache->capacity;
  a.cv = cache_view(cache);
  a.hkv = n_kv_heads;
  a.hd = head_dim;
  a.elem = es;
  a.prefix_len = prefix_len;
  a.h_nodes = h_nodes;
  a.hidden = hidden;
  a.next_feature = next_feature;
  a.max_accept = max_accept;
  a.accept_len = accept_len;
  a.path = path;
  a.out_tokens = out_tokens;
  a.next_token = next_token;
  a.status = dev_status;
  return EAGLE_OK;
}

// ---- scratch of the entry point that allocates nothing ---------------------------------
// One copy of this array exists on every GPU the library runs on, from the first use on
// that GPU until the process ends.  In host code its name is only a stand-in: the device
// address is taken once per device with hipGetSymbolAddress and kept in scratch_dev[].
static __device__ __align__(256) unsigned char scratch[EAGLE_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first call there).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return EAGLE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EAGLE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EAGLE_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return EAGLE_OK;
}
}  // namespace

}  // namespace eagle

using namespace eagle;

extern "C" {

int eagle_abi_version(void) { return EAGLE_ABI_VERSION; }

const char* eagle_status_str(int st) {
  switch (st) {
    case EAGLE_OK: return "ok";
    case EAGLE_ERR_ARG: return "invalid argument";
    case EAGLE_ERR_TREE: return "malformed parent array";
    case EAGLE_ERR_CAPACITY: return "capacity exceeded";
    case EAGLE_ERR_UNSUPPORTED: return "unsupported dimensions";
    case EAGLE_ERR_HIP: return "HIP error";
    case EAGLE_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int eagle_tree_build(int32_t batch, const int32_t* tree_off, int32_t total_nodes, int32_t max_nodes,
                     const int32_t* parent, const int32_t* prefix_len, int32_t mask_words, uint64_t* anc,
                     int32_t* depth, int32_t* pos, int32_t* dev_status, void* stream) {
  if (batch < 1 || total_nodes < 1 || max_nodes < 1) return EAGLE_ERR_ARG;
  if (!tree_off || !parent || !prefix_len || !anc || !depth || !pos) return EAGLE_ERR_ARG;
  if (mask_words < 1 || mask_words > 2) return EAGLE_ERR_UNSUPPORTED;
  if (max_nodes > 64 * mask_words) return EAGLE_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  return launch_tree_build(batch, tree_off, parent, prefix_len, mask_words, max_nodes, total_nodes, anc, depth, pos,
                           dev_status, s);
}

int eagle_tree_verify(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln, const void* w_lm,
                      int32_t batch, const int32_t* tree_off, int32_t total_nodes, int32_t max_nodes,
                      const void* x_in, const void* embed, const int32_t* tokens, const uint64_t* anc,
                      int32_t mask_words, const int32_t* pos, const int32_t* prefix_len, int32_t max_prefix,
                      const void* k_cache, const void* v_cache, const eagle_cache_layout* cache, void* k_tree,
                      void* v_tree, float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn,
                      float* dbg_logits, void* workspace, size_t ws_bytes, eagle_timer* timer, void* stream) {
  return verify_impl(dims, layer, 1, 0, final_ln, w_lm, batch, tree_off, total_nodes, max_nodes, x_in, embed,
                     tokens, anc, mask_words, pos, prefix_len, max_prefix, k_cache, v_cache, cache, k_tree, v_tree,
                     h_out, argmax, maxlogit, dbg_attn, dbg_logits, workspace, ws_bytes, timer, (hipStream_t)stream);
}

int eagle_tree_verify_noalloc(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln,
                              const void* w_lm, int32_t batch, const int32_t* tree_off, int32_t total_nodes,
                              int32_t max_nodes, const void* x_in, const void* embed, const int32_t* tokens,
                              const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                              const int32_t* prefix_len, int32_t max_prefix, const void* k_cache,
                              const void* v_cache, const eagle_cache_layout* cache, void* k_tree, void* v_tree,
                              float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn, float* dbg_logits,
                              eagle_timer* timer, void* stream) {
  return verify_impl(dims, layer, 1, 0, final_ln, w_lm, batch, tree_off, total_nodes, max_nodes, x_in, embed,
                     tokens, anc, mask_words, pos, prefix_len, max_prefix, k_cache, v_cache, cache, k_tree, v_tree,
                     h_out, argmax, maxlogit, dbg_attn, dbg_logits, nullptr, EAGLE_NOALLOC_MAX_BYTES, timer,
                     (hipStream_t)stream, nullptr, scratch_ptr);
}

int eagle_tree_verify_layers(const eagle_dims* dims, int32_t n_layers, const eagle_layer_w* layers,
                             const void* final_ln, const void* w_lm, int32_t batch, const int32_t* tree_off,
                             int32_t total_nodes, int32_t max_nodes, const void* x_in, const void* embed,
                             const int32_t* tokens, const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                             const int32_t* prefix_len, int32_t max_prefix, const void* k_cache, const void* v_cache,
                             const eagle_cache_layout* cache, int64_t cache_layer_stride, void* k_tree,
                             void* v_tree, float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn,
                             float* dbg_logits, void* workspace, size_t ws_bytes, eagle_timer* timer, void* stream) {
  return verify_impl(dims, layers, n_layers, cache_layer_stride, final_ln, w_lm, batch, tree_off, total_nodes,
                     max_nodes, x_in, embed, tokens, anc, mask_words, pos, prefix_len, max_prefix, k_cache, v_cache,
                     cache, k_tree, v_tree, h_out, argmax, maxlogit, dbg_attn, dbg_logits, workspace, ws_bytes, timer,
                     (hipStream_t)stream);
}

int eagle_accept_commit(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                        const int32_t* tokens, const int32_t* argmax, const uint64_t* anc, int32_t mask_words,
                        const int32_t* depth, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                        const eagle_cache_layout* cache, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t* prefix_len, const float* h_nodes, int32_t hidden, float* next_feature,
                        int32_t max_accept, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                        int32_t* next_token, int32_t* dev_status, void* stream) {
  if (!argmax || !anc || !depth) return EAGLE_ERR_ARG;
  if (mask_words < 1 || mask_words > 2 || max_nodes > 64 * mask_words) return EAGLE_ERR_CAPACITY;
  AcceptArgs a{};
  const int rc = commit_args(a, batch, tree_off, max_nodes, parent, tokens, k_tree, v_tree, k_cache, v_cache, cache,
                             n_kv_heads, head_dim, dtype, prefix_len, h_nodes, hidden, next_feature, max_accept,
                             accept_len, path, out_tokens, next_token, dev_status);
  if (rc) return rc;
  a.argmax = argmax;
  a.anc = anc;
  a.mw = mask_words;
  a.depth = depth;
  return launch_accept_commit(a, batch, (hipStream_t)stream);
}

int eagle_accept_commit_layers(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                               const int32_t* tokens, const int32_t* argmax, const uint64_t* anc,
                               int32_t mask_words, const int32_t* depth, const void* k_tree, const void* v_tree,
                               void* k_cache, void* v_cache, const eagle_cache_layout* cache, int32_t n_kv_heads,
                               int32_t head_dim, int32_t dtype, int32_t n_layers, int64_t cache_layer_stride,
                               int64_t tree_layer_stride, int32_t* prefix_len, const float* h_nodes,
                               int32_t hidden, float* next_feature, int32_t max_accept, int32_t* accept_len,
                               int32_t* path, int32_t* out_tokens, int32_t* next_token, int32_t* dev_status,
                               void* stream) {
  if (!argmax || !anc || !depth) return EAGLE_ERR_ARG;
  if (mask_words < 1 || mask_words > 2 || max_nodes > 64 * mask_words) return EAGLE_ERR_CAPACITY;
  if (n_layers < 1 || n_layers > 1024) return EAGLE_ERR_ARG;
  if (n_layers > 1 && (cache_layer_stride <= 0 || tree_layer_stride <= 0)) return EAGLE_ERR_ARG;
  AcceptArgs a{};
  int rc = commit_args(a, batch, tree_off, max_nodes, parent, tokens, k_tree, v_tree, k_cache, v_cache, cache,
                       n_kv_heads, head_dim, dtype, prefix_len, h_nodes, hidden, next_feature, max_accept,
                       accept_len, path, out_tokens, next_token, dev_status);
  if (rc) return rc;
  const int es = elem_size(dtype);
  if ((cache_layer_stride * es) % 16 || (tree_layer_stride * es) % 16) return EAGLE_ERR_ARG;
  a.argmax = argmax;
  a.anc = anc;
  a.mw = mask_words;
  a.depth = depth;
  a.n_layers = n_layers;
  a.cache_ls = cache_layer_stride;
  a.tree_ls = tree_layer_stride;
  rc = launch_accept_commit(a, batch, (hipStream_t)stream);
  if (rc) return rc;
  return launch_commit_layers(a, batch, (hipStream_t)stream);
}

int eagle_accept_commit_sample(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                               const int32_t* tokens, const float* child_logit, const float* rest_lse,
                               const int32_t* rest_token, const float* u, const void* k_tree, const void* v_tree,
                               void* k_cache, void* v_cache, const eagle_cache_layout* cache, int32_t n_kv_heads,
                               int32_t head_dim, int32_t dtype, int32_t* prefix_len, const float* h_nodes,
                               int32_t hidden, float* next_feature, int32_t max_accept, int32_t* accept_len,
                               int32_t* path, int32_t* out_tokens, int32_t* next_token, int32_t* dev_status,
                               void* stream) {
  if (!child_logit || !rest_lse || !rest_token || !u) return EAGLE_ERR_ARG;
  if (max_nodes > 128) return EAGLE_ERR_CAPACITY;
  AcceptArgs a{};
  const int rc = commit_args(a, batch, tree_off, max_nodes, parent, tokens, k_tree, v_tree, k_cache, v_cache, cache,
                             n_kv_heads, head_dim, dtype, prefix_len, h_nodes, hidden, next_feature, max_accept,
                             accept_len, path, out_tokens, next_token, dev_status);
  if (rc) return rc;
  a.child_logit = child_logit;
  a.rest_lse = rest_lse;
  a.rest_token = rest_token;
  a.u = u;
  return launch_accept_sample(a, batch, (hipStream_t)stream);
}

int eagle_tree_verify_sample(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln,
                             const void* w_lm, int32_t batch, const int32_t* tree_off, int32_t total_nodes,
                             int32_t max_nodes, const void* x_in, const void* embed, const int32_t* tokens,
                             const int32_t* parent, const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                             const int32_t* prefix_len, int32_t max_prefix, const void* k_cache,
                             const void* v_cache, const eagle_cache_layout* cache, float temperature,
                             const float* gumbel, void* k_tree, void* v_tree, float* h_out, float* child_logit,
                             float* rest_lse, int32_t* rest_token, void* workspace, size_t ws_bytes,
                             eagle_timer* timer, void* stream) {
  SampleOut so{parent, temperature, gumbel, child_logit, rest_lse, rest_token};
  return verify_impl(dims, layer, 1, 0, final_ln, w_lm, batch, tree_off, total_nodes, max_nodes, x_in, embed,
                     tokens, anc, mask_words, pos, prefix_len, max_prefix, k_cache, v_cache, cache, k_tree, v_tree,
                     h_out, nullptr, nullptr, nullptr, nullptr, workspace, ws_bytes, timer, (hipStream_t)stream, &so);
}

size_t eagle_workspace_size(int32_t which, const eagle_dims* dims, int32_t batch, int32_t total_nodes,
                            int32_t max_nodes, int32_t max_prefix, const eagle_draft_params* params) {
  if (which == 0) return verify_workspace(dims, batch, total_nodes, max_nodes, max_prefix);
  if (which == 1) return draft_workspace(dims, params, batch, max_prefix);
  if (which == 2) return fuse_layout(dims, batch).total;
  if (which == 3) return verify_workspace(dims, batch, total_nodes, max_nodes, max_prefix, true);
  if (which == 4) return draft_kv_workspace(dims, batch, max_nodes - 1);
  return 0;
}

int eagle_fuse_features(const eagle_dims* dims, const void* w_fuse, int32_t w_layout, const void* feats,
                        int32_t batch, float* root_feature, void* workspace, size_t ws_bytes, void* stream) {
  if (!dims || !w_fuse || !feats || !root_feature || !workspace || batch < 1) return EAGLE_ERR_ARG;
  if (w_layout != 0 && w_layout != 1) return EAGLE_ERR_ARG;
  if (((uintptr_t)workspace) & 255) return EAGLE_ERR_ARG;
  if (dims->dtype != EAGLE_BF16 || dims->hidden <= 0 || dims->hidden % 64) return EAGLE_ERR_UNSUPPORTED;
  const FuseLayout L = fuse_layout(dims, batch);
  if (ws_bytes < L.total) return EAGLE_ERR_WORKSPACE;
  const int H = dims->hidden;
  char* w = (char*)workspace;
  GemmDesc g{};
  g.dtype = EAGLE_BF16;
  g.w0 = w_fuse;
  g.w_layout = w_layout;
  g.n = H;
  g.k = 3 * H;
  g.ldw = 3 * H;
  g.m = batch;
  g.x.a = seg(feats, EAGLE_BF16, 3 * H);
  g.x.b = g.x.a;
  g.x.ka = 3 * H;
  g.epi.kind = EPI_STORE_F32;
  g.epi.out = root_feature;
  g.epi.ld_out = H;
  g.partials = (float*)(w + L.part);
  g.sumsq_part = (float*)(w + L.ssq);
  g.counters = (int*)(w + L.counters);
  return launch_gemm(g, L.plan, (hipStream_t)stream);
}

int eagle_pack_fragments(const void* w, int32_t rows, int32_t cols, void* out, void* stream) {
  if (!w || !out || rows <= 0 || cols <= 0 || cols % 32) return EAGLE_ERR_ARG;
  if (((uintptr_t)w | (uintptr_t)out) % 16) return EAGLE_ERR_ARG;
  eagle::launch_pack_fragments(w, rows, cols, out, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int eagle_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace) return EAGLE_ERR_ARG;
  return launch_fill_zero(workspace, ws_bytes, (hipStream_t)stream);
}

eagle_timer* eagle_timer_create(int32_t capacity) {
  if (capacity < 1) return nullptr;
  eagle_timer* t = new eagle_timer();
  t->cap = capacity;
  t->ev.resize(2 * capacity);
  t->stage.resize(capacity);
  for (auto& e : t->ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      delete t;
      return nullptr;
    }
  }
  return t;
}

void eagle_timer_destroy(eagle_timer* t) {
  if (!t) return;
  for (auto& e : t->ev) (void)hipEventDestroy(e);  // nothing to do on failure at teardown
  delete t;
}

int eagle_timer_select(eagle_timer* t, uint32_t stage_mask) {
  if (!t) return EAGLE_ERR_ARG;
  t->mask = stage_mask;
  return EAGLE_OK;
}

int eagle_timer_collect(eagle_timer* t, double* ms, int32_t* count) {
  if (!t || !ms || !count) return EAGLE_ERR_ARG;
  for (int i = 0; i < t->n; ++i) {
    if (hipEventSynchronize(t->ev[2 * i + 1]) != hipSuccess) return EAGLE_ERR_HIP;
    float e = 0.f;
    if (hipEventElapsedTime(&e, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess) return EAGLE_ERR_HIP;
    const int st = t->stage[i];
    if (st >= 0 && st < EAGLE_N_STAGES) {
      ms[st] += e;
      count[st] += 1;
    }
  }
  t->n = 0;
  t->open = false;
  return EAGLE_OK;
}

}  // extern "C"
