// Internal interface of the tree encode and accept/commit kernels.
#pragma once

#include "common.h"

namespace eagle {

struct AcceptArgs {
  const int32_t* tree_off;
  const int32_t* parent;
  const int32_t* tokens;
  const int32_t* argmax;
  const uint64_t* anc;
  int mw;
  const int32_t* depth;
  const void* k_tree;
  const void* v_tree;
  void* k_cache;
  void* v_cache;
  CacheView cv;  // cache addressing (contiguous or paged)
  int capacity;
  int hkv, hd, elem;
  int32_t* prefix_len;
  const float* h_nodes;
  int hidden;
  float* next_feature;
  int max_accept;
  int32_t* accept_len;
  int32_t* path;
  int32_t* out_tokens;
  int32_t* next_token;
  int32_t* status;
  // acceptance at temperature T > 0 (argmax, anc, mw and depth unused): per node the
  // tempered logit of its token under its parent, the log-normaliser and best noisy
  // token of its non-child tokens, and its acceptance uniform
  const float* child_logit;
  const float* rest_lse;
  const int32_t* rest_token;
  const float* u;
  // commit of a layer stack (commit_layers_kernel): layer l's tree K/V start at
  // l * tree_ls elements of k_tree/v_tree and its caches at l * cache_ls elements
  int n_layers;
  int64_t cache_ls, tree_ls;
};

int launch_tree_build(int batch, const int32_t* tree_off, const int32_t* parent, const int32_t* prefix_len, int mw,
                      int max_nodes, int total_nodes, uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* status,
                      hipStream_t s);
int launch_accept_commit(const AcceptArgs& a, int batch, hipStream_t s);
int launch_sample_prep(const int32_t* tree_off, const int32_t* parent, int batch, int total, int32_t* gparent,
                       int32_t* row_tree, hipStream_t s);
int launch_sample_merge(const float4* part, int n_part, int rows, float* rest_lse, int32_t* rest_token,
                        hipStream_t s);
int launch_accept_sample(const AcceptArgs& a, int batch, hipStream_t s);
// Layers 1 .. n_layers-1 of a stack, after launch_accept_commit committed layer 0.
int launch_commit_layers(const AcceptArgs& a, int batch, hipStream_t s);

}  // namespace eagle
