// Tree encode and greedy accept + KV commit (gfx950).
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
                                                         const int32_t* prefix_len, int mw, uint64_t* anc,
                                                         int32_t* depth, int32_t* pos, int32_t* status) {
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int off = tree_off[b];
  const int N = tree_off[b + 1] - off;
  if (threadIdx.x == 0) s_bad = (N < 1 || N > 64 * mw) ? EAGLE_ERR_CAPACITY : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < N && !s_bad; i += blockDim.x) {
    const int p = parent[off + i];
    if ((i == 0 && p != -1) || (i > 0 && (p < 0 || p >= i))) atomicCAS(&s_bad, 0, EAGLE_ERR_TREE);
  }
  __syncthreads();
  const int bad = s_bad;
  if (bad) {
    if (threadIdx.x == 0) set_status(status, bad);
    for (int i = threadIdx.x; i < N * mw && bad == EAGLE_ERR_TREE; i += blockDim.x) anc[(int64_t)off * mw + i] = 0ull;
    return;
  }
  const int P = prefix_len[b];
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    uint64_t words[2] = {0ull, 0ull};
    int d = 0;
    int j = i;
    // parent[j] < j for every non-root node, so the walk ends at the root in <= i steps
    while (true) {
      words[j >> 6] |= 1ull << (j & 63);
      if (j == 0) break;
      j = parent[off + j];
      ++d;
    }
    for (int w = 0; w < mw; ++w) anc[(int64_t)(off + i) * mw + w] = words[w];
    depth[off + i] = d;
    pos[off + i] = P + d;
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
  __shared__ int s_L, s_leaf, s_P, s_ok;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int off = a.tree_off[b];
  const int N = a.tree_off[b + 1] - off;
  const int mw = a.mw;
  if (N < 1 || N > 64 * mw || N > NMAX) {
    if (tid == 0) {
      set_status(a.status, EAGLE_ERR_CAPACITY);
      a.accept_len[b] = -1;
      a.next_token[b] = -1;
    }
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
  }
  __syncthreads();
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
  const int stride = a.max_accept + 1;
  if (!s_ok) {
    if (tid == 0) {
      a.accept_len[b] = -1;
      a.next_token[b] = -1;
    }
    for (int d = tid; d < stride; d += blockDim.x) {
      a.path[(int64_t)b * stride + d] = -1;
      a.out_tokens[(int64_t)b * stride + d] = -1;
    }
    return;
  }
  // path: ancestors of the leaf have increasing index and depth, so node j on the path
  // sits at position depth[j]
  for (int j = tid; j < N; j += blockDim.x) {
    const int dj = s_dep[j];
    if (((s_anc[leaf][j >> 6] >> (j & 63)) & 1ull) && dj >= 0 && dj <= L) s_path[dj] = j;
  }
  __syncthreads();
  const int bonus = s_am[leaf];
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
  // commit K/V rows of path[0..L] into slots P..P+L (16-byte copies; rows are
  // hd * elem bytes, a multiple of 16)
  const int row_bytes = a.hd * a.elem;
  const int chunks = row_bytes / 16;
  const int per_node = a.hkv * chunks;
  const int total = (L + 1) * per_node;
  for (int i = tid; i < 2 * total; i += blockDim.x) {
    const int which = i / total;  // 0: K, 1: V
    const int r = i % total;
    const int d = r / per_node;
    const int h = (r % per_node) / chunks;
    const int ch = r % chunks;
    const char* src = (const char*)(which ? a.v_tree : a.k_tree) +
                      ((int64_t)(off + s_path[d]) * a.hkv + h) * row_bytes + ch * 16;
    char* dst = (char*)(which ? a.v_cache : a.k_cache) +
                ((int64_t)b * a.cb + (int64_t)h * a.ch + (int64_t)(P + d) * a.ct) * a.elem + ch * 16;
    *(uint4*)dst = *(const uint4*)src;
  }
  if (a.next_feature) {
    for (int i = tid * 4; i < a.hidden; i += blockDim.x * 4)
      *(float4*)(a.next_feature + (int64_t)b * a.hidden + i) =
          *(const float4*)(a.h_nodes + (int64_t)(off + leaf) * a.hidden + i);
  }
  if (tid == 0) a.prefix_len[b] = P + L + 1;
}

}  // namespace

int launch_tree_build(int batch, const int32_t* tree_off, const int32_t* parent, const int32_t* prefix_len, int mw,
                      uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(tree_build_kernel, dim3(batch), dim3(128), 0, s, tree_off, parent, prefix_len, mw, anc, depth,
                     pos, status);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

int launch_accept_commit(const AcceptArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(accept_commit_kernel, dim3(batch), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP;
}

}  // namespace eagle
