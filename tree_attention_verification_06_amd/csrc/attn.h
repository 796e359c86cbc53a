// Internal interface of the tree-masked GQA attention kernels.
#pragma once

#include "common.h"

namespace eagle {

struct AttnArgs {
  int dtype;  // EAGLE_BF16 (MFMA path, head_dim 128) or EAGLE_F32 (VALU path)
  int batch, hq, hkv, hd;
  const void* q;         // [sum N][hq][hd]
  const void* k_cache;   // cache layout below
  const void* v_cache;
  int64_t cb, ch, ct;    // cache strides (elements); cb is the page stride when paged
  int cap;               // cache slots per (b, h); prefix lengths are clamped to it
  const int32_t* table;  // paged cache: block table [B][maxb] (nullptr: contiguous)
  int ps, maxb, npages;  // page size, table entries per sequence, pages in the pool
  const void* k_tree;    // [sum N][hkv][hd]
  const void* v_tree;
  const uint64_t* anc;   // [sum N][mw]
  int mw;
  const int32_t* tree_off;
  const int32_t* prefix_len;
  int max_nodes, max_prefix;  // max_nodes bounds the query nodes of a sequence
  // Optional query subset (draft levels): sequence b has n_nodes[b] key nodes starting at
  // tree_off[b]; only nodes q_lo[b] .. n_nodes[b]-1 are queries, and their q / output rows
  // are b * q_stride + (node - q_lo[b]).  nullptr / 0: every node is a query and its row is
  // tree_off[b] + node, with n_nodes = tree_off[b+1] - tree_off[b].
  const int32_t* n_nodes;
  const int32_t* q_lo;
  int q_stride;
  void* out;             // [sum N][hq * hd] (dtype)
  float* dbg;            // optional [sum N][hq * hd] f32
  // split-KV plan and partials (bf16 path)
  int kch, n_chunks;     // prefix chunk length; chunks including the tree chunk
  int row_groups;        // groups of query rows (16 per wave) per (b, kv head)
  float* part_o;         // [B][hkv][n_chunks][rmax][hd]
  float* part_ml;        // [B][hkv][n_chunks][rmax][2]
};

struct AttnPlan {
  int kch, n_chunks, row_groups, rmax;
  int nwa;  // waves per workgroup of the bf16 kernel (4 or 8)
};

AttnPlan plan_attn(int dtype, int batch, int hq, int hkv, int hd, int max_nodes, int max_prefix);
size_t attn_workspace_floats(const AttnPlan& p, int batch, int hkv, int hd);
int launch_attn(AttnArgs& a, const AttnPlan& p, eagle_timer* timer, hipStream_t s);
int launch_attn_f32(AttnArgs& a, int total_nodes, eagle_timer* timer, hipStream_t s);

}  // namespace eagle
