// Tree encode, acceptance (greedy, and sampling at T > 0) + KV commit (gfx950).
//
// Both are integer work on at most 128 nodes per tree, so each tree gets one
// workgroup and each node one lane: ancestor words are built by walking the parent
// chain, and the accept step is a handful of ballots over the match bits followed by
// a cooperative 16-byte copy of the accepted K/V rows into the cache.
#include "common.h"
#include "tree.h"

namespace eagle {

namespace {

__device__ __forceinline__ void set_status(int32_t* st, int code) {
  if (st) atomicCAS(st, 0, code);
}

// One workgroup (128 threads) per tree; node i handled by thread i, i + 128, ...
__global__ __launch_bounds__(128) void tree_build_kernel(const int32_t* tree_off, const int32_t* parent,
                                                         const int32_t* prefix_len, int mw, int max_nodes,
                                                         int total_nodes, uint64_t* anc, int32_t* depth,
                                                         int32_t* pos, int32_t* status) {
  // the tree's parent array is staged in LDS (one round of loads) and every ancestor walk
  // runs there, instead of one dependent global load per level of depth
  __shared__ int s_bad;
  __shared__ int s_par[128];
  const int b = blockIdx.x;
  const int off = tree_off[b];
  const int N = tree_off[b + 1] - off;
  const int P = prefix_len[b];  // (requested with the offsets: one round trip fewer)
  // a tree outside the caller's rows, or larger than the mask words or max_nodes (which
  // sizes the attention grid) is refused and nothing of it is written
  if (threadIdx.x == 0)
    s_bad = (off < 0 || N < 1 || off + N > total_nodes || N > 64 * mw || N > 128 || N > max_nodes)
                ? EAGLE_ERR_CAPACITY
                : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < N && !s_bad; i += blockDim.x) {
    const int p = parent[off + i];
    s_par[i] = p;
    if ((i == 0 && p != -1) || (i > 0 && (p < 0 || p >= i))) atomicCAS(&s_bad, 0, EAGLE_ERR_TREE);
  }
  __syncthreads();
  const int bad = s_bad;
  if (bad) {
    if (threadIdx.x == 0) set_status(status, bad);
    for (int i = threadIdx.x; i < N * mw && bad == EAGLE_ERR_TREE; i += blockDim.x) anc[(int64_t)off * mw + i] = 0ull;
    return;
  }
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    uint64_t words[2] = {0ull, 0ull};
    int d = 0;
    int j = i;
    // parent[j] < j for every non-root node, so the walk ends at the root in <= i steps
    while (true) {
      words[j >> 6] |= 1ull << (j & 63);
      if (j == 0) break;
      j = s_par[j];
      ++d;
    }
    for (int w = 0; w < mw; ++w) anc[(int64_t)(off + i) * mw + w] = words[w];
    depth[off + i] = d;
    pos[off + i] = P + d;
  }
}

// Outputs and commit of sequence b, shared by both acceptance rules: path and
// out_tokens for the accepted path s_path[0..L] (LDS) and the bonus token, then the K/V
// rows of the path into cache slots P..P+L (16-byte copies; rows are hd * elem bytes,
// a multiple of 16), the leaf's feature into next_feature, and prefix_len[b] = P + L + 1.
// Every thread of the workgroup calls it.
__device__ void commit_path(const AcceptArgs& a, int b, int off, const int* s_path, const int* s_tok, int L, int leaf,
                            int bonus, int P) {
  const int tid = threadIdx.x;
  const int stride = a.max_accept + 1;
  for (int d = tid; d < stride; d += blockDim.x) {
    a.path[(int64_t)b * stride + d] = d <= L ? s_path[d] : -1;
    int t = -1;
    if (d < L) t = s_tok[s_path[d + 1]];
    else if (d == L) t = bonus;
    a.out_tokens[(int64_t)b * stride + d] = t;
  }
  if (tid == 0) {
    a.accept_len[b] = L;
    a.next_token[b] = bonus;
  }
  // 16-byte pieces: the K and V rows of the path and the leaf's feature.  Loads are
  // issued in batches before their stores (a load-store pair per piece would cost one
  // memory round trip each: the stores may alias later loads), and a thread's indices
  // are formed once, without a division per piece (integer division is tens of VALU
  // instructions, which at one workgroup per sequence cost as much as a round trip).
  const int nthr = blockDim.x;
  const int row_bytes = a.hd * a.elem;
  const int chunks = row_bytes / 16;
  const int per_node = a.hkv * chunks;  // pieces of one node's K (or V) rows
  const int nf = a.next_feature ? a.hidden / 4 : 0;
  const f32x4* feat_src = (const f32x4*)(a.h_nodes + (int64_t)(off + leaf) * a.hidden);
  f32x4* feat_dst = (f32x4*)(a.next_feature + (int64_t)b * a.hidden);
  // the first four feature pieces of this thread are requested ahead of the K/V rows
  constexpr int UF = 4;
  f32x4 fv[UF];
  if (nf > 0) {
#pragma unroll
    for (int u = 0; u < UF; ++u) fv[u] = feat_src[min(tid + u * nthr, nf - 1)];
  }
  if (per_node <= nthr) {
    // thread: piece j of a node's rows (head h, chunk ch) for the path depths d = g,
    // g + G, ... (G groups of per_node threads), K and V together, DU depths per round
    const int G = nthr / per_node;
    const int g = tid / per_node, jn = tid - g * per_node;
    const int h = jn / chunks, ch = jn - h * chunks;
    const char* kt = (const char*)a.k_tree + (int64_t)h * row_bytes + ch * 16;
    const char* vt = (const char*)a.v_tree + (int64_t)h * row_bytes + ch * 16;
    const int64_t node_bytes = (int64_t)a.hkv * row_bytes;
    constexpr int DU = 4;
    if (g < G) {
      for (int d0 = g; d0 <= L; d0 += DU * G) {
        f32x4 kv[DU][2];
        int64_t co[DU];
        bool st[DU];
#pragma unroll
        for (int u = 0; u < DU; ++u) {
          const int d = d0 + u * G;
          const int dc = min(d, L);  // past the path: re-read its last node, store nothing
          const int64_t src = (int64_t)(off + s_path[dc]) * node_bytes;
          kv[u][0] = *(const f32x4*)(kt + src);
          kv[u][1] = *(const f32x4*)(vt + src);
          bool ok;
          co[u] = cache_offset(a.cv, b, h, P + dc, ok);
          st[u] = d <= L && ok;
          if (d <= L && !ok) set_status(a.status, EAGLE_ERR_ARG);  // a bad page id: never written through
        }
#pragma unroll
        for (int u = 0; u < DU; ++u)
          if (st[u]) {
            *(f32x4*)((char*)a.k_cache + co[u] * a.elem + ch * 16) = kv[u][0];
            *(f32x4*)((char*)a.v_cache + co[u] * a.elem + ch * 16) = kv[u][1];
          }
      }
    }
  } else {
    // wide rows (more pieces per node than threads): one piece per iteration
    const int total = (L + 1) * per_node;
    for (int i = tid; i < 2 * total; i += nthr) {
      const int which = i / total;  // 0: K, 1: V
      const int r = i - which * total;
      const int d = r / per_node;
      const int h = (r - d * per_node) / chunks;
      const int ch = r % chunks;
      const char* src = (const char*)(which ? a.v_tree : a.k_tree) +
                        ((int64_t)(off + s_path[d]) * a.hkv + h) * row_bytes + ch * 16;
      bool ok;
      const int64_t co = cache_offset(a.cv, b, h, P + d, ok);
      if (!ok) {  // a bad page id: never written through
        set_status(a.status, EAGLE_ERR_ARG);
        continue;
      }
      *(f32x4*)((char*)(which ? a.v_cache : a.k_cache) + co * a.elem + ch * 16) = *(const f32x4*)src;
    }
  }
  if (nf > 0) {
#pragma unroll
    for (int u = 0; u < UF; ++u)
      if (tid + u * nthr < nf) feat_dst[tid + u * nthr] = fv[u];
    for (int f0 = tid + UF * nthr; f0 < nf; f0 += UF * nthr) {
#pragma unroll
      for (int u = 0; u < UF; ++u) fv[u] = feat_src[min(f0 + u * nthr, nf - 1)];
#pragma unroll
      for (int u = 0; u < UF; ++u)
        if (f0 + u * nthr < nf) feat_dst[f0 + u * nthr] = fv[u];
    }
  }
  if (tid == 0) a.prefix_len[b] = P + L + 1;
}

// A sequence that cannot be accepted: accept_len and next_token -1, path and
// out_tokens all -1, nothing committed.
__device__ void reject_sequence(const AcceptArgs& a, int b) {
  const int stride = a.max_accept + 1;
  if (threadIdx.x == 0) {
    a.accept_len[b] = -1;
    a.next_token[b] = -1;
  }
  for (int d = threadIdx.x; d < stride; d += blockDim.x) {
    a.path[(int64_t)b * stride + d] = -1;
    a.out_tokens[(int64_t)b * stride + d] = -1;
  }
}

// One workgroup (256 threads) per sequence.  Every per-node array of the tree is read
// into LDS in a single round of independent loads; the match / consistency / leaf /
// path logic then runs in LDS, and all output stores and K/V copies go out together.
__global__ __launch_bounds__(256) void accept_commit_kernel(AcceptArgs a) {
  constexpr int NMAX = 128;
  __shared__ int s_tok[NMAX], s_par[NMAX], s_dep[NMAX], s_am[NMAX];
  __shared__ uint64_t s_anc[NMAX][2];
  __shared__ uint64_t s_match[2];
  __shared__ unsigned long long s_best;
  __shared__ int s_path[NMAX + 1];
  __shared__ int s_L, s_leaf, s_P, s_ok, s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int off = a.tree_off[b];
  const int N = a.tree_off[b + 1] - off;
  const int mw = a.mw;
  if (N < 1 || N > 64 * mw || N > NMAX) {
    if (tid == 0) set_status(a.status, EAGLE_ERR_CAPACITY);
    reject_sequence(a, b);
    return;
  }
  for (int i = tid; i < N; i += blockDim.x) {
    s_tok[i] = a.tokens[off + i];
    s_par[i] = a.parent[off + i];
    s_dep[i] = a.depth[off + i];
    s_am[i] = a.argmax[off + i];
    s_anc[i][0] = a.anc[(int64_t)(off + i) * mw];
    s_anc[i][1] = mw > 1 ? a.anc[(int64_t)(off + i) * mw + 1] : 0ull;
  }
  for (int i = tid; i <= NMAX; i += blockDim.x) s_path[i] = 0;
  if (tid < 2) s_match[tid] = 0ull;
  if (tid == 0) {
    s_best = 0ull;
    s_P = a.prefix_len[b];
    s_bad = 0;
  }
  __syncthreads();
  // the tree must be well formed (parent[0] = -1, parent[i] in [0, i)) and its depth and
  // ancestor words must be the encoding of that parent array: a malformed tree leaves them
  // zeroed or stale, and a stale depth would otherwise pick a leaf and commit a path
  for (int i = tid; i < N; i += blockDim.x) {
    const int p = s_par[i];
    bool bad;
    if (i == 0) {
      bad = p != -1 || s_dep[0] != 0 || s_anc[0][0] != 1ull || s_anc[0][1] != 0ull;
    } else {
      bad = p < 0 || p >= i;
      if (!bad) {
        const uint64_t self0 = (i >> 6) == 0 ? 1ull << (i & 63) : 0ull;
        const uint64_t self1 = (i >> 6) == 1 ? 1ull << (i & 63) : 0ull;
        bad = s_dep[i] != s_dep[p] + 1 || s_anc[i][0] != (s_anc[p][0] | self0) || s_anc[i][1] != (s_anc[p][1] | self1);
      }
    }
    if (bad) atomicCAS(&s_bad, 0, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) set_status(a.status, EAGLE_ERR_TREE);
    reject_sequence(a, b);
    return;
  }
  // match bits: the root always matches; node j matches iff its token is the target's
  // argmax at its parent
  for (int i = tid; i < N; i += blockDim.x) {
    bool m = true;
    if (i > 0) {
      const int p = s_par[i];
      m = p >= 0 && p < i && s_tok[i] == s_am[p];
    }
    if (m) atomicOr((unsigned long long*)&s_match[i >> 6], 1ull << (i & 63));
  }
  __syncthreads();
  // consistent nodes: every node on the root path matches; pick the deepest, lowest index
  for (int i = tid; i < N; i += blockDim.x) {
    const bool ok = ((s_anc[i][0] & ~s_match[0]) == 0ull) && ((s_anc[i][1] & ~s_match[1]) == 0ull);
    if (ok) {
      const unsigned long long key =
          ((unsigned long long)(uint32_t)s_dep[i] << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
      atomicMax(&s_best, key);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int leaf = (int)(0xffffffffu - (uint32_t)(s_best & 0xffffffffull));
    const int L = (int)(s_best >> 32);
    s_leaf = leaf;
    s_L = L;
    const bool fits = L <= a.max_accept && s_P >= 0 && (int64_t)s_P + L + 1 <= a.capacity;
    s_ok = fits;
    if (!fits) set_status(a.status, EAGLE_ERR_CAPACITY);
  }
  __syncthreads();
  const int L = s_L, leaf = s_leaf, P = s_P;
  if (!s_ok) {
    reject_sequence(a, b);
    return;
  }
  // path: ancestors of the leaf have increasing index and depth, so node j on the path
  // sits at position depth[j]
  for (int j = tid; j < N; j += blockDim.x) {
    const int dj = s_dep[j];
    if (((s_anc[leaf][j >> 6] >> (j & 63)) & 1ull) && dj >= 0 && dj <= L) s_path[dj] = j;
  }
  __syncthreads();
  commit_path(a, b, off, s_path, s_tok, L, leaf, s_am[leaf], P);
}


// ---- acceptance at temperature T > 0 ----------------------------------------------

// Global parent row of every row (-1: a root, a padding row past tree_off[B] or a
// malformed parent) and the sequence each row belongs to (-1: padding).  Workgroup b
// < batch handles tree b, workgroup `batch` the padding rows.
__global__ __launch_bounds__(128) void sample_prep_kernel(const int32_t* tree_off, const int32_t* parent, int batch,
                                                          int total, int32_t* gparent, int32_t* row_tree) {
  const int b = blockIdx.x;
  if (b == batch) {
    for (int r = max(tree_off[batch], 0) + threadIdx.x; r < total; r += blockDim.x) {
      gparent[r] = -1;
      row_tree[r] = -1;
    }
    return;
  }
  const int off = tree_off[b];
  const int N = tree_off[b + 1] - off;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int r = off + i;
    if (r < 0 || r >= total) continue;
    const int p = parent[r];
    gparent[r] = (i > 0 && p >= 0 && p < i) ? off + p : -1;
    row_tree[r] = b;
  }
}

__device__ __forceinline__ void lse_combine(float& M, float& S, float m2, float s2) {
  const float Mn = fmaxf(M, m2);
  if (Mn == -INFINITY) return;  // both empty
  S = (M == -INFINITY ? 0.f : S * __expf(M - Mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - Mn));
  M = Mn;
}

// Row m of the LM head's per-tile summaries -> rest_lse[m] = log sum exp over the row's
// non-child tokens and rest_token[m] = the token of the largest noisy key.  One
// workgroup per row; its n_part entries are contiguous and read in one round.
__global__ __launch_bounds__(256) void sample_merge_kernel(const float4* part, int n_part, float* rest_lse,
                                                           int32_t* rest_token) {
  constexpr int R = 4;
  __shared__ float s_m[4], s_s[4];
  __shared__ unsigned long long s_k[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float4* p = part + (int64_t)m * n_part;
  float M = -INFINITY, S = 0.f;
  unsigned long long K = 0ull;
  for (int i0 = tid; i0 < n_part; i0 += R * 256) {
    float4 q[R];
#pragma unroll
    for (int u = 0; u < R; ++u) q[u] = p[min(i0 + u * 256, n_part - 1)];  // in-range stand-in past the end
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (i0 + u * 256 >= n_part) continue;
      lse_combine(M, S, q[u].x, q[u].y);
      const unsigned long long k2 =
          ((unsigned long long)__float_as_uint(q[u].w) << 32) | (unsigned long long)__float_as_uint(q[u].z);
      K = k2 > K ? k2 : K;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(M, o, 64), s2 = __shfl_xor(S, o, 64);
    const unsigned long long k2 = __shfl_xor(K, o, 64);
    lse_combine(M, S, m2, s2);
    K = k2 > K ? k2 : K;
  }
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    s_m[w] = M;
    s_s[w] = S;
    s_k[w] = K;
  }
  __syncthreads();
  if (tid == 0) {
    for (int j = 1; j < 4; ++j) {
      lse_combine(M, S, s_m[j], s_s[j]);
      K = s_k[j] > K ? s_k[j] : K;
    }
    rest_lse[m] = M == -INFINITY ? -INFINITY : M + __logf(S);
    rest_token[m] = K ? (int32_t)(0xffffffffu - (uint32_t)(K & 0xffffffffull)) : -1;
  }
}

// One workgroup (256 threads) per sequence.  The walk is sequential by nature (a child
// is tried only once its elder siblings are rejected), so wave 0 runs it over LDS copies
// of the tree: at each visited node two ballots over the parent array give its children
// in index order, a wave reduction combines rest_lse with the children's logits into the
// node's log-normaliser, and the children are then tried in turn.  The other waves only
// help with the loads, the checks and the commit.
__global__ __launch_bounds__(256) void accept_sample_kernel(AcceptArgs a) {
  constexpr int NMAX = 128;
  __shared__ int s_tok[NMAX], s_par[NMAX], s_rt[NMAX];
  __shared__ float s_z[NMAX], s_rl[NMAX], s_u[NMAX];
  __shared__ int s_path[NMAX + 1];
  __shared__ int s_L, s_leaf, s_bonus, s_P, s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int off = a.tree_off[b];
  const int N = a.tree_off[b + 1] - off;
  if (N < 1 || N > NMAX) {
    if (tid == 0) set_status(a.status, EAGLE_ERR_CAPACITY);
    reject_sequence(a, b);
    return;
  }
  for (int i = tid; i < N; i += blockDim.x) {
    s_tok[i] = a.tokens[off + i];
    s_par[i] = a.parent[off + i];
    s_z[i] = a.child_logit[off + i];
    s_rl[i] = a.rest_lse[off + i];
    s_rt[i] = a.rest_token[off + i];
    s_u[i] = a.u[off + i];
  }
  if (tid == 0) {
    s_P = a.prefix_len[b];
    s_bad = 0;
  }
  __syncthreads();
  // a well-formed tree (parent[0] = -1, parent[i] in [0, i)) with distinct sibling tokens
  for (int i = tid; i < N; i += blockDim.x) {
    const int p = s_par[i];
    bool bad = (i == 0) ? p != -1 : (p < 0 || p >= i);
    if (!bad && i > 0)
      for (int j = p + 1; j < i; ++j) bad |= s_par[j] == p && s_tok[j] == s_tok[i];
    if (bad) atomicCAS(&s_bad, 0, 1);
  }
  __syncthreads();
  if (tid < 64 && !s_bad) {
    const int lane = tid;
    int node = 0, L = 0, bonus = -1;
    while (true) {
      if (lane == 0) s_path[L] = node;
      const int c0 = lane, c1 = lane + 64;
      const bool k0 = c0 > node && c0 < N && s_par[c0] == node;
      const bool k1 = c1 > node && c1 < N && s_par[c1] == node;
      const unsigned long long b0 = __ballot(k0), b1 = __ballot(k1);
      const float z0 = k0 ? s_z[c0] : -INFINITY, z1 = k1 ? s_z[c1] : -INFINITY;
      const float rl = s_rl[node];
      const float mz = fmaxf(rl, wave_max(fmaxf(z0, z1)));
      const float sz = wave_sum((k0 ? __expf(z0 - mz) : 0.f) + (k1 ? __expf(z1 - mz) : 0.f));
      const float lse = mz + __logf((rl == -INFINITY ? 0.f : __expf(rl - mz)) + sz);
      float r = 1.f;  // mass left after the rejected children
      int next = -1;
      for (int w = 0; w < 2 && next < 0; ++w) {
        unsigned long long bits = w ? b1 : b0;
        while (bits) {
          const int c = w * 64 + __builtin_ctzll(bits);
          bits &= bits - 1;
          const float px = __expf(s_z[c] - lse);
          if (s_u[c] * r < px) {
            next = c;
            break;
          }
          r -= px;
        }
      }
      if (next < 0) {
        bonus = s_rt[node];
        break;
      }
      node = next;
      ++L;
    }
    if (lane == 0) {
      s_L = L;
      s_leaf = node;
      s_bonus = bonus;
    }
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) set_status(a.status, EAGLE_ERR_TREE);
    reject_sequence(a, b);
    return;
  }
  const int L = s_L, P = s_P;
  if (L > a.max_accept || P < 0 || (int64_t)P + L + 1 > a.capacity) {
    if (tid == 0) set_status(a.status, EAGLE_ERR_CAPACITY);
    reject_sequence(a, b);
    return;
  }
  commit_path(a, b, off, s_path, s_tok, L, s_leaf, s_bonus, P);
}

}  // namespace

int launch_tree_build(int batch, const int32_t* tree_off, const int32_t* parent, const int32_t* prefix_len, int mw,
                      int max_nodes, int total_nodes, uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* status,
                      hipStream_t s) {
  hipLaunchKernelGGL(tree_build_kernel, dim3(batch), dim3(128), 0, s, tree_off, parent, prefix_len, mw, max_nodes,
                     total_nodes, anc, depth, pos, status);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

// Commit of the layers above the first in a stack of decoder layers.  accept_commit_kernel
// has already chosen the path, committed layer 0 and advanced prefix_len, so workgroup
// (b, l - 1) reads accept_len[b] and path[b] and copies layer l's tree K/V of the path into
// that layer's cache slots P .. P + L with P = prefix_len[b] - L - 1.  A rejected sequence
// (accept_len -1) is skipped.  Each thread issues up to eight independent 16-byte loads
// before its stores, so the copy is not one load latency per chunk.
__global__ __launch_bounds__(256) void commit_layers_kernel(AcceptArgs a) {
  const int b = blockIdx.x, l = blockIdx.y + 1;
  const int L = a.accept_len[b];
  if (L < 0) return;
  const int P = a.prefix_len[b] - L - 1;
  const int off = a.tree_off[b];
  const int stride = a.max_accept + 1;
  const int row_bytes = a.hd * a.elem;
  const int chunks = row_bytes / 16;
  const int per_node = a.hkv * chunks;
  const int total = 2 * (L + 1) * per_node;
  const char* kt = (const char*)a.k_tree + (size_t)l * a.tree_ls * a.elem;
  const char* vt = (const char*)a.v_tree + (size_t)l * a.tree_ls * a.elem;
  char* kc = (char*)a.k_cache + (size_t)l * a.cache_ls * a.elem;
  char* vc = (char*)a.v_cache + (size_t)l * a.cache_ls * a.elem;
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < total; i0 += U * blockDim.x) {
    f32x4 v[U];  // (16 raw bytes; a vector type keeps the array in registers)
    char* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * blockDim.x;
      dst[u] = nullptr;
      if (i < total) {
        const int which = i / (total / 2);  // 0: K, 1: V
        const int r = i % (total / 2);
        const int d = r / per_node;
        const int h = (r % per_node) / chunks;
        const int ch = r % chunks;
        const int node = a.path[(int64_t)b * stride + d];
        v[u] = *(const f32x4*)((which ? vt : kt) + ((int64_t)(off + node) * a.hkv + h) * row_bytes + ch * 16);
        bool ok;
        const int64_t co = cache_offset(a.cv, b, h, P + d, ok);
        if (ok)
          dst[u] = (which ? vc : kc) + co * a.elem + ch * 16;
        else
          set_status(a.status, EAGLE_ERR_ARG);  // a bad page id: never written through
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u]) *(f32x4*)dst[u] = v[u];
  }
}

int launch_commit_layers(const AcceptArgs& a, int batch, hipStream_t s) {
  if (a.n_layers < 2) return EAGLE_OK;
  hipLaunchKernelGGL(commit_layers_kernel, dim3(batch, a.n_layers - 1), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_accept_commit(const AcceptArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(accept_commit_kernel, dim3(batch), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_sample_prep(const int32_t* tree_off, const int32_t* parent, int batch, int total, int32_t* gparent,
                       int32_t* row_tree, hipStream_t s) {
  hipLaunchKernelGGL(sample_prep_kernel, dim3(batch + 1), dim3(128), 0, s, tree_off, parent, batch, total, gparent,
                     row_tree);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_sample_merge(const float4* part, int n_part, int rows, float* rest_lse, int32_t* rest_token,
                        hipStream_t s) {
  hipLaunchKernelGGL(sample_merge_kernel, dim3(rows), dim3(256), 0, s, part, n_part, rest_lse, rest_token);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_accept_sample(const AcceptArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(accept_sample_kernel, dim3(batch), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle
