/*
 * eagle.h - C ABI of an MI355X (gfx950) library for the hot path of EAGLE
 * feature-level speculative decoding: the tree-verification step and the
 * draft head's tree expansion.
 *
 * Method sources (web pages; cited by page title and section):
 *  - "Speculative decoding with EAGLE" (aiunderstanding.org), Deep dive and
 *    Technical insight: a cheap drafter proposes candidate tokens; the target
 *    checks all of them in a single parallel pass and keeps the longest
 *    correct prefix; accepted tokens must equal the target's own (argmax)
 *    choice, so the output equals what the target produces alone; the drafter
 *    predicts hidden features, is fed the true embedding of the previous
 *    token, and reuses the target's LM head.
 *  - "LLM parallel decoding EAGLE" (jisaku.com glossary), How EAGLE works:
 *    one-layer decoder draft head over the final hidden features; several
 *    candidate tokens per predicted feature expanded into a tree; tree
 *    attention verifies every node in one forward pass and the longest valid
 *    path is accepted.  EAGLE vs EAGLE-2 table: a fixed 60-node topology
 *    (EAGLE-1) or confidence-adaptive trees of 40..120 nodes (EAGLE-2).
 *    FAQ Q3: pruning at a confidence threshold of 0.3.
 *
 * Conventions shared by every call
 *  - All pointers are DEVICE pointers unless a parameter says "host".  All
 *    device buffers are allocated and freed by the caller; the library never
 *    allocates device memory and keeps no pointer after a call returns.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *    default stream) and never synchronises.  Buffers must stay valid until
 *    the stream has executed the work.
 *  - Weights are row-major [out][in] (each output row contiguous over the
 *    input dimension).  bf16 tensors are IEEE bfloat16; f32 tensors are IEEE
 *    binary32.  The element type of weights, activations given as `void*`,
 *    KV caches and tree K/V is `eagle_dims.dtype`.
 *  - Trees of a batch are concatenated: tree b owns nodes
 *    tree_off[b] .. tree_off[b+1]-1 of every per-node array.  Parent indices
 *    are local to their tree; node 0 of each tree is the root (parent -1) and
 *    0 <= parent[i] < i for every other node.  The root is the last committed
 *    token (the previous step's bonus token), whose K/V is not in the cache
 *    yet, so it is verified and committed together with the accepted nodes.
 *  - KV caches are [B][Hkv][capacity][D] with the strides given in
 *    eagle_cache_layout (elements; d is contiguous).  Slots 0..prefix_len[b]-1
 *    of sequence b hold its committed keys (already rotated) and values.
 *  - Return value: EAGLE_OK or a negative eagle_status for argument errors
 *    detectable on the host; nothing is enqueued in that case.  Errors that
 *    depend on device data (a malformed parent array, cache overflow) are
 *    written to `dev_status` (first error wins; the caller zeroes it) and the
 *    affected sequence's outputs are left as documented per call.
 *  - Workspace: a caller-owned device buffer of at least
 *    eagle_workspace_size() bytes, 256-byte aligned, zero-filled once after
 *    allocation (eagle_workspace_init).  Every call leaves the synchronisation
 *    counters it uses back at zero, so the same workspace can be reused
 *    without clearing.  Calls that share one workspace must not overlap.
 */
#ifndef EAGLE_H_
#define EAGLE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EAGLE_ABI_VERSION 7

typedef enum {
  EAGLE_OK = 0,
  EAGLE_ERR_ARG = -1,         /* null pointer, bad size, misaligned buffer */
  EAGLE_ERR_TREE = -2,        /* malformed parent array (device-side)       */
  EAGLE_ERR_CAPACITY = -3,    /* tree or accepted path exceeds a capacity   */
  EAGLE_ERR_UNSUPPORTED = -4, /* dims outside what the kernels implement    */
  EAGLE_ERR_HIP = -5,         /* a HIP launch or runtime call failed        */
  EAGLE_ERR_WORKSPACE = -6    /* workspace too small                        */
} eagle_status;

typedef enum { EAGLE_BF16 = 0, EAGLE_F32 = 1 } eagle_dtype;

/* Shape of one decoder layer and its LM head.
 *  ffn == 0 and rms_eps == 0 select the attention-only layer:
 *    y = x + W_o attn(x),  logits = W_lm y   (no norms, no MLP).
 *  Otherwise the Llama-style pre-norm layer:
 *    y = x + W_o attn(RMSNorm(x)),  h = y + W_down(SiLU(W_gate y') * W_up y'),
 *    y' = RMSNorm(y),  logits = W_lm RMSNorm(h).
 *  rope_theta == 0 disables the rotary embedding; otherwise q and k are rotated
 *  in the rotate-half pairing (j, j + D/2) with angle pos * theta^(-2j/D).
 *  Supported: bf16 with head_dim 128; f32 with head_dim 64 or 128;
 *  n_q_heads a multiple of n_kv_heads; hidden a multiple of 64. */
typedef struct {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rope_theta, rms_eps;
  int32_t dtype;     /* eagle_dtype */
  int32_t lm_layout; /* layout of w_lm: 0 row-major [V][H]; 1 fragment-blocked as written
                        by eagle_pack_fragments (bf16 only).  Same arithmetic either way. */
} eagle_dims;

/* Weights of one decoder layer (element type dims.dtype).  The matrices are [rows][cols]
 * as listed, row-major when layout == 0, or each in the fragment-blocked layout written by
 * eagle_pack_fragments when layout == 1 (bf16 only; the same arithmetic either way).  For
 * a draft layer, layout also applies to its w_fc. */
typedef struct {
  const void* ln_attn; /* [H] RMSNorm gain before attention (NULL if rms_eps == 0) */
  const void* w_qkv;   /* [(Hq + 2 Hkv) D][H]: q rows (head-major), then k rows, then v rows */
  const void* w_o;     /* [H][Hq D] */
  const void* ln_mlp;  /* [H] RMSNorm gain before the MLP (NULL if ffn == 0) */
  const void* w_gate;  /* [F][H] */
  const void* w_up;    /* [F][H] */
  const void* w_down;  /* [H][F] */
  int32_t layout;      /* 0 row-major, 1 fragment-blocked */
} eagle_layer_w;

/* KV cache geometry, in elements.
 * Contiguous (block_table == NULL): element (b, h, t, d) is at
 *   b*batch_stride + h*head_stride + t*token_stride + d.
 * Paged (block_table != NULL), for continuous batching: the cache is a pool of n_pages
 * pages of page_size token slots each, and sequence b owns the pages listed in
 * block_table[b * max_blocks .. + max_blocks - 1] (device int32): element (b, h, t, d) is at
 *   block_table[b*max_blocks + t/page_size]*batch_stride + h*head_stride
 *     + (t % page_size)*token_stride + d,
 * i.e. batch_stride is the page stride.  page_size must be a positive multiple of 64
 * and capacity <= max_blocks * page_size (else EAGLE_ERR_ARG).  Pages may be shared by
 * no two sequences that are written.  A page id outside [0, n_pages) is read as page
 * n_pages - 1 or 0 (no fault; the values are meaningless) and is never written: a
 * commit that would write through it sets *dev_status = EAGLE_ERR_ARG and skips that
 * row.  The same table serves every layer of a stack (the layer stride moves the pool). */
typedef struct {
  int64_t batch_stride, head_stride, token_stride;
  int32_t capacity; /* slots per (b, h) */
  const int32_t* block_table;
  int32_t page_size, max_blocks, n_pages;
} eagle_cache_layout;

/* Draft expansion parameters (readings of the pages' EAGLE-2 description). */
typedef struct {
  int32_t depth;        /* expansion levels (1..16)                                   */
  int32_t top_k;        /* children per expanded node (1..16)                         */
  int32_t frontier;     /* nodes expanded per level after the first (1..16)           */
  int32_t max_nodes;    /* final tree size per sequence, root included (2..128)       */
  float conf_threshold; /* a child is expandable iff its probability >= this, [0, 1]  */
} eagle_draft_params;

/* ---- EAGLE-3 draft input ----------------------------------------------------
 * Method: "LLM parallel decoding EAGLE" (EAGLE vs EAGLE-2 table and FAQ: EAGLE-3 feeds
 * the draft a fusion of the target's low-, mid- and high-level features rather than its
 * top feature) and the "yuhuili" author page (EAGLE-3).  The pages give no formula; the
 * reading here is one linear map with no bias:
 *   root_feature[b] = W_fuse [f_low[b]; f_mid[b]; f_high[b]]
 * after which eagle_draft_expand runs unchanged on root_feature (its FC takes
 * [root_feature; E[root token]] at the first level).
 * Inputs: w_fuse [H][3H] bf16, row-major (w_layout 0) or fragment-blocked (w_layout 1,
 * eagle_pack_fragments); feats [batch][3H] bf16, the three features of each sequence
 * concatenated.  Output: root_feature [batch][H] f32 (fp32 accumulation).
 * Workspace: eagle_workspace_size(2, dims, batch, 0, 0, 0, NULL) bytes, zero-filled once.
 * Errors: NULL pointers, batch < 1, w_layout not 0/1, misaligned workspace -> ARG;
 * dims not bf16 or hidden not a multiple of 64 -> UNSUPPORTED; small workspace -> WORKSPACE. */
int eagle_fuse_features(const eagle_dims* dims, const void* w_fuse, int32_t w_layout, const void* feats,
                        int32_t batch, float* root_feature, void* workspace, size_t ws_bytes, void* stream);

/* ---- weight packing ------------------------------------------------------
 * A layout of this library (the pages prescribe none): a fragment-blocked copy of
 * a row-major bf16 matrix W [rows][cols], cols a positive multiple of 32.  With
 * nblk = ceil(rows / 16), the 8 elements of lane l (0..63) of 16-row block b at
 * 32-column step s start at element ((s * nblk + b) * 64 + l) * 8 of out and hold
 * W[16 b + l % 16][32 s + 8 (l / 16) .. 32 s + 8 (l / 16) + 7] (zeros for rows past
 * the last).  These are the bf16 MFMA A operands in the order the GEMMs consume
 * them; all blocks of one step are contiguous, so a GEMM whose workgroups advance
 * through K together streams one compact region at a time.
 * Inputs: w (device, 16-byte aligned); out (device, 16-byte aligned, nblk * 16 *
 * cols elements, caller-owned, must not overlap w).  Asynchronous on stream.
 * Errors: NULL or misaligned pointers, rows <= 0 or a bad cols -> EAGLE_ERR_ARG. */
int eagle_pack_fragments(const void* w, int32_t rows, int32_t cols, void* out, void* stream);

/* ---- tree encode -------------------------------------------------------
 * Method: "LLM parallel decoding EAGLE", How EAGLE works (tree attention: a
 * node sees the prefix and its own root path).  For every node i of tree b:
 *   depth[i] = depth[parent[i]] + 1 (root 0);
 *   anc[i][w] bit j set iff node 64w+j of the same tree is i or an ancestor of i;
 *   pos[i] = prefix_len[b] + depth[i].
 * tree_off [B+1], parent [total_nodes], prefix_len [B] are inputs;
 * anc [total_nodes][mask_words] (uint64), depth and pos [total_nodes] outputs.
 * Host: total_nodes >= tree_off[B] (rows past tree_off[B] are padding and are
 * not touched), max_nodes >= every tree size, both host ints.
 * Errors: mask_words*64 < max_nodes -> EAGLE_ERR_CAPACITY (host).  A tree with
 * parent[0] != -1 or parent[i] outside [0, i) sets *dev_status = EAGLE_ERR_TREE
 * and its anc words are all zero (depth/pos then undefined).  A tree of more than
 * max_nodes nodes, or reaching past total_nodes, sets *dev_status =
 * EAGLE_ERR_CAPACITY and nothing of it is written. */
int eagle_tree_build(int32_t batch, const int32_t* tree_off, int32_t total_nodes, int32_t max_nodes,
                     const int32_t* parent, const int32_t* prefix_len, int32_t mask_words,
                     uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* dev_status, void* stream);

/* ---- tree verification --------------------------------------------------
 * Method: "Speculative decoding with EAGLE", Deep dive (all drafted tokens
 * checked in one parallel pass) and "LLM parallel decoding EAGLE", How EAGLE
 * works (tree attention).  One decoder layer over every node of every tree:
 *   x = x_in (or embed[tokens] when x_in is NULL), node positions pos;
 *   attention of node i: softmax(q_i k_j / sqrt(D)) over every prefix slot of
 *   its sequence and over the tree nodes set in anc[i] (GQA: query head h uses
 *   KV head h / (Hq/Hkv));
 *   h_out = layer output (the next draft feature), argmax[i] = first index of
 *   the maximum of logits_i = W_lm RMSNorm(h_i), maxlogit[i] = that maximum.
 *   The [total_nodes][vocab] logits are never written (unless dbg_logits).
 * Inputs: x_in [total_nodes][H] (dtype) or NULL; embed [V][H] or NULL; tokens
 * [total_nodes]; anc [total_nodes][mask_words]; pos [total_nodes]; prefix_len
 * [B]; k_cache/v_cache (read only).  Host ints: total_nodes, max_nodes,
 * max_prefix (sizes the split of the prefix over workgroups; a prefix_len[b] above
 * it is still attended in full, by the last split, only more slowly; prefix_len is
 * clamped to the cache capacity).  total_nodes may
 * exceed tree_off[B]: rows past it are padding, computed row by row and never
 * attended to (their tokens must still be valid ids when x_in is NULL).
 * Outputs: k_tree, v_tree [total_nodes][Hkv][D] (dtype; post-rotary keys),
 * h_out [total_nodes][H] f32, argmax [total_nodes] i32, maxlogit [total_nodes] f32.
 * Optional outputs (NULL to skip): dbg_attn [total_nodes][Hq D] f32 attention
 * output, dbg_logits [total_nodes][V] f32 full logits.
 * The cache is not modified, so verification can be repeated freely.
 * timer: optional (NULL), records per-kernel HIP events (eagle_timer_*). */
typedef struct eagle_timer eagle_timer;

int eagle_tree_verify(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln,
                      const void* w_lm, int32_t batch, const int32_t* tree_off, int32_t total_nodes,
                      int32_t max_nodes, const void* x_in, const void* embed, const int32_t* tokens,
                      const uint64_t* anc, int32_t mask_words, const int32_t* pos, const int32_t* prefix_len,
                      int32_t max_prefix, const void* k_cache, const void* v_cache,
                      const eagle_cache_layout* cache, void* k_tree, void* v_tree, float* h_out,
                      int32_t* argmax, float* maxlogit, float* dbg_attn, float* dbg_logits,
                      void* workspace, size_t ws_bytes, eagle_timer* timer, void* stream);

/* eagle_tree_verify_noalloc: eagle_tree_verify for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments minus workspace and ws_bytes, same arithmetic,
 * outputs and host errors.  Its scratch is a buffer of EAGLE_NOALLOC_MAX_BYTES (32 MiB)
 * inside the library: one copy per GPU, held from the first call on that GPU until the
 * process ends.  A call whose eagle_workspace_size(0, ...) exceeds that returns
 * EAGLE_ERR_WORKSPACE and enqueues nothing (the 8B layer with one 60-node tree and
 * max_prefix 2048 needs 21 MiB; the 70B layer or batch-16 shapes do not fit: use
 * eagle_tree_verify with a workspace).  Every call on a GPU uses the same buffer, so calls
 * that overlap on one GPU (different streams, threads or processes sharing no order) race
 * and give wrong results; calls ordered on one stream are fine.  Each call clears the
 * counters it needs with a fill kernel (no memset node).  The first call on each device
 * resolves the buffer's address (hipGetSymbolAddress, no allocation); make it outside
 * graph capture.  Errors: as eagle_tree_verify; EAGLE_ERR_HIP if the address cannot be
 * resolved. */
#define EAGLE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int eagle_tree_verify_noalloc(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln,
                              const void* w_lm, int32_t batch, const int32_t* tree_off, int32_t total_nodes,
                              int32_t max_nodes, const void* x_in, const void* embed, const int32_t* tokens,
                              const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                              const int32_t* prefix_len, int32_t max_prefix, const void* k_cache,
                              const void* v_cache, const eagle_cache_layout* cache, void* k_tree, void* v_tree,
                              float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn, float* dbg_logits,
                              eagle_timer* timer, void* stream);

/* ---- acceptance and KV commit -------------------------------------------
 * Method: "Speculative decoding with EAGLE", Deep dive and FAQ (keep the
 * longest correct prefix; accepted tokens equal the target's choice, hence
 * lossless); "LLM parallel decoding EAGLE", How EAGLE works (the longest valid
 * path is accepted).  Greedy rule per tree b:
 *   match(j) = tokens[j] == argmax[parent(j)] for non-root j;
 *   a node is consistent iff every non-root node on its root path matches;
 *   leaf = deepest consistent node (ties: lowest index), L = depth[leaf];
 *   path[b][0..L] = root .. leaf, out_tokens[b][0..L] = tokens of path[1..L]
 *   followed by the bonus token argmax[leaf]; next_token[b] = argmax[leaf];
 *   accept_len[b] = L.
 * Commit: cache slot prefix_len[b] + d <- (k_tree, v_tree) of path[d] for
 * d = 0..L, then prefix_len[b] += L + 1; next_feature[b] = h_nodes[leaf].
 * The copies read k_tree/v_tree, never the cache, so there is no in-place hazard.
 * Inputs: tree_off, parent, tokens, argmax, anc, depth, k_tree, v_tree, h_nodes
 * [total_nodes][hidden] f32.  In/out: k_cache, v_cache, prefix_len.
 * Outputs: accept_len [B], path and out_tokens [B][max_accept + 1] (entries
 * past L are -1), next_token [B], next_feature [B][hidden] f32 (NULL to skip).
 * Device errors: L > max_accept or prefix_len + L + 1 > capacity set
 * *dev_status = EAGLE_ERR_CAPACITY; a malformed parent array, or depth / anc
 * that are not its encoding (e.g. left zeroed or stale by a failed
 * eagle_tree_build), sets *dev_status = EAGLE_ERR_TREE; such a sequence gets
 * accept_len -1, next_token -1, path and out_tokens all -1 and no commit. */
int eagle_accept_commit(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                        const int32_t* tokens, const int32_t* argmax, const uint64_t* anc, int32_t mask_words,
                        const int32_t* depth, const void* k_tree, const void* v_tree, void* k_cache,
                        void* v_cache, const eagle_cache_layout* cache, int32_t n_kv_heads, int32_t head_dim,
                        int32_t dtype, int32_t* prefix_len, const float* h_nodes, int32_t hidden,
                        float* next_feature, int32_t max_accept, int32_t* accept_len, int32_t* path,
                        int32_t* out_tokens, int32_t* next_token, int32_t* dev_status, void* stream);

/* ---- verification and acceptance at temperature T > 0 ---------------------
 * Method: "Speculative decoding with EAGLE", Deep dive and FAQ (the accepted
 * tokens follow the target's own distribution, so decoding is lossless).  The
 * pages give no sampling procedure; the reading implemented is speculative
 * sampling with the tree's tokens as deterministic candidates, walked from the
 * root: at node n with p = softmax(logits_n / T), its children c are tried in
 * index order; c is accepted iff u[c] * r < p(tokens[c]), r being the mass left
 * once the tokens of the rejected elder siblings are removed (r = 1 at first);
 * on acceptance the walk moves to c.  When every child of n is rejected (or n is
 * a leaf) the bonus token is drawn from p without n's child tokens by the
 * Gumbel-max rule, argmax_v (log p(v) + gumbel[b][v]).  Each emitted token is
 * then distributed as the target's p at its position.  Exactly one bonus is
 * drawn per sequence and where it is drawn depends on u only, so the noise row
 * gumbel[b] is shared by every node of tree b.  Sibling tokens must be distinct.
 *
 * eagle_tree_verify_sample: the decoder layer of eagle_tree_verify (same
 * arguments, plus parent [total_nodes] local parents and tokens required), then
 * the LM head summarised per node n (v = logits_n / T):
 *   child_logit[c] = v_{parent(c)}[tokens[c]] for every non-root node c (the
 *   root's entry is not written);
 *   rest_lse[n] = log sum_v exp(v) over the tokens that are not a child token of n;
 *   rest_token[n] = argmax over the same tokens of v + gumbel[b][token] (ties:
 *   the lower id), b the tree of n.
 * The [total_nodes][vocab] logits are never written.  gumbel [B][V] f32 standard
 * Gumbel noise (device).  temperature > 0 and finite 1/T, else EAGLE_ERR_ARG.
 * Rows past tree_off[B] are computed and meaningless.  Workspace:
 * eagle_workspace_size(3, ...). */
int eagle_tree_verify_sample(const eagle_dims* dims, const eagle_layer_w* layer, const void* final_ln,
                             const void* w_lm, int32_t batch, const int32_t* tree_off, int32_t total_nodes,
                             int32_t max_nodes, const void* x_in, const void* embed, const int32_t* tokens,
                             const int32_t* parent, const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                             const int32_t* prefix_len, int32_t max_prefix, const void* k_cache,
                             const void* v_cache, const eagle_cache_layout* cache, float temperature,
                             const float* gumbel, void* k_tree, void* v_tree, float* h_out, float* child_logit,
                             float* rest_lse, int32_t* rest_token, void* workspace, size_t ws_bytes,
                             eagle_timer* timer, void* stream);

/* eagle_accept_commit_sample: the walk above per tree b from the outputs of
 * eagle_tree_verify_sample: the log-normaliser of node n is the log-sum-exp of
 * rest_lse[n] and the child_logit of its children; p(tokens[c]) =
 * exp(child_logit[c] - that); the bonus of the node where the walk stops is
 * rest_token[n].  u [total_nodes] uniforms in [0, 1), u[c] decides node c.
 * Outputs and commit exactly as eagle_accept_commit (path root..leaf,
 * out_tokens = accepted tokens then the bonus, next_token = the bonus,
 * next_feature = h_nodes[leaf]).  Host errors as eagle_accept_commit, and
 * max_nodes > 128 -> EAGLE_ERR_CAPACITY.  Device errors: a tree of more than 128
 * nodes -> EAGLE_ERR_CAPACITY; parent[0] != -1, parent[i] outside [0, i) or two
 * siblings with the same token -> EAGLE_ERR_TREE; L > max_accept or no cache
 * room -> EAGLE_ERR_CAPACITY; such a sequence gets accept_len -1 and no commit. */
int eagle_accept_commit_sample(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                               const int32_t* tokens, const float* child_logit, const float* rest_lse,
                               const int32_t* rest_token, const float* u, const void* k_tree, const void* v_tree,
                               void* k_cache, void* v_cache, const eagle_cache_layout* cache, int32_t n_kv_heads,
                               int32_t head_dim, int32_t dtype, int32_t* prefix_len, const float* h_nodes,
                               int32_t hidden, float* next_feature, int32_t max_accept, int32_t* accept_len,
                               int32_t* path, int32_t* out_tokens, int32_t* next_token, int32_t* dev_status,
                               void* stream);

/* ---- draft-head tree expansion -------------------------------------------
 * Method: "Speculative decoding with EAGLE", Technical insight (feature-level
 * draft head fed the true previous-token embedding; reuses the target LM
 * head); "LLM parallel decoding EAGLE", How EAGLE works (one-layer decoder head,
 * candidates expanded into a tree), EAGLE vs EAGLE-2 table and FAQ Q3
 * (confidence-adaptive trees, pruning threshold).  Level-synchronous, per
 * sequence b, starting from the root (root_token[b], feature root_feature[b]):
 *   draft row of node n = W_fc [f_parent(n) ; embed[token n]] (f_parent of the
 *   root = root_feature[b]) -> the draft decoder layer at position
 *   prefix_len[b] + depth(n), attending to the draft KV prefix and the expanded
 *   draft nodes on n's root path (itself included) -> feature f_hat(n);
 *   log p = log_softmax(W_lm RMSNorm_final(f_hat(n))) over the vocabulary; the
 *   top_k tokens (ties: lower id) become children with
 *   cum = cum(n) + min(0, log p) (cum(root) = 0);
 *   children with log p >= log(conf_threshold) are expandable; the next level
 *   expands the `frontier` best expandable children by (cum desc, generation
 *   order asc), generation order = (level, parent rank, child rank).
 * After `depth` levels the tree is the root plus the best max_nodes-1 candidates
 * by (cum desc, depth asc, generation order asc), re-indexed by (depth asc, cum
 * desc, generation order asc); cum never grows along a path, so the kept set
 * contains every kept node's parent.
 * Weights: w_fc [H][2H] (feature columns first), draft_layer (all seven
 * tensors), the target's final_ln [H] and w_lm [V][H], embed [V][H]; all bf16.
 * Inputs: root_feature [B][H] f32, root_token [B], dk_cache/dv_cache (the draft
 * layer's own KV prefix, post-rotary keys, read only), prefix_len [B]; host int
 * max_prefix >= every prefix_len[b].
 * Outputs: tree_off [B+1]; parent, tokens [B*max_nodes] i32 and cum_logp
 * [B*max_nodes] f32.  Tree b occupies [tree_off[b], tree_off[b+1]) with local
 * parent indices (root first, parent -1).  A tree has fewer than max_nodes nodes
 * only when pruning leaves fewer candidates; entries from tree_off[B] up to
 * B*max_nodes are then padding (parent -1, token 0, cum -inf), so the arrays can
 * go straight into eagle_tree_verify with total_nodes = B*max_nodes and no
 * host synchronisation (padding rows are computed and ignored).
 * Supported: dtype bf16, head_dim 128, a normed layer (ffn > 0, rms_eps > 0),
 * top_k and frontier in 1..16, 1 + (depth-1)*frontier <= 64,
 * 1 + top_k + (depth-1)*frontier*top_k <= 2048, frontier*top_k <= 256.
 * The workspace (eagle_workspace_size(1, ...)) must be zero-filled once
 * (eagle_workspace_init) and not shared with a concurrent call. */
int eagle_draft_expand(const eagle_dims* dims, const eagle_draft_params* params, const void* w_fc,
                       const eagle_layer_w* draft_layer, const void* final_ln, const void* w_lm,
                       const void* embed, int32_t batch, const float* root_feature, const int32_t* root_token,
                       const void* dk_cache, const void* dv_cache, const eagle_cache_layout* cache,
                       const int32_t* prefix_len, int32_t max_prefix, int32_t* tree_off, int32_t* parent,
                       int32_t* tokens, float* cum_logp, void* workspace, size_t ws_bytes,
                       eagle_timer* timer, void* stream);

/* Candidate pool of the last eagle_draft_expand that used this workspace (same
 * dims, params, batch, max_prefix), for inspection.  Per sequence b, with
 * P = 1 + top_k + (depth-1)*frontier*top_k: pool_n[b] candidates in generation
 * order (root first, then each level's children by parent frontier rank and
 * child rank); token, parent (pool index, -1 for the root), depth [B][P] i32,
 * cum_logp and logp (the child's own log-probability; 0 for the root) [B][P]
 * f32, entries past pool_n[b] are -1 / -inf; expanded [B][depth][frontier] i32
 * = pool indices expanded on each level (-1 padded).  Any output may be NULL. */
int eagle_draft_pool(const eagle_dims* dims, const eagle_draft_params* params, int32_t batch,
                     int32_t max_prefix, const void* workspace, size_t ws_bytes, int32_t* pool_n,
                     int32_t* token, int32_t* parent, int32_t* depth, float* cum_logp, float* logp,
                     int32_t* expanded, void* stream);

/* ---- a target of several decoder layers, and the draft KV update --------------
 * Method: "Speculative decoding with EAGLE", Deep dive (the target verifies every
 * drafted token in one pass; the emitted text is what the target alone would produce)
 * and Technical insight (the draft works on the target's hidden features and is fed the
 * true embedding of the next token); "yuhuili" page (the draft reads the target's
 * second-top-layer features).  The pages describe a full model; the readings here: the
 * target is n_layers Llama-style layers (eagle_dims, ffn > 0 and rms_eps > 0) applied in
 * order, each with its own KV cache, under one final norm and LM head; every layer sees
 * the same tree mask and positions; a node's feature is the last layer's output.
 *
 * eagle_tree_verify_layers: eagle_tree_verify through layers[0 .. n_layers-1] (host
 * array of n_layers eagle_layer_w; layer l's input is layer l-1's output h, f32).
 * Caches: layer l's cache is at k_cache/v_cache + l * cache_layer_stride elements (each
 * layer [B][Hkv][capacity][D] with the strides of `cache`).  Outputs: k_tree, v_tree
 * [n_layers][total_nodes][Hkv][D] (layer l at l * total_nodes * Hkv * D elements),
 * h_out = the last layer's output, argmax/maxlogit of the LM head on it; dbg_attn (NULL to
 * skip) is the last layer's attention output.  n_layers == 1 is eagle_tree_verify.
 * Errors: as eagle_tree_verify; n_layers outside 1..1024 or a negative stride ->
 * EAGLE_ERR_ARG; n_layers > 1 without the MLP layer -> EAGLE_ERR_UNSUPPORTED.
 * Workspace: eagle_workspace_size(0, ...), the same as one layer (buffers are reused). */
int eagle_tree_verify_layers(const eagle_dims* dims, int32_t n_layers, const eagle_layer_w* layers,
                             const void* final_ln, const void* w_lm, int32_t batch, const int32_t* tree_off,
                             int32_t total_nodes, int32_t max_nodes, const void* x_in, const void* embed,
                             const int32_t* tokens, const uint64_t* anc, int32_t mask_words, const int32_t* pos,
                             const int32_t* prefix_len, int32_t max_prefix, const void* k_cache, const void* v_cache,
                             const eagle_cache_layout* cache, int64_t cache_layer_stride, void* k_tree,
                             void* v_tree, float* h_out, int32_t* argmax, float* maxlogit, float* dbg_attn,
                             float* dbg_logits, void* workspace, size_t ws_bytes, eagle_timer* timer, void* stream);

/* eagle_accept_commit_layers: eagle_accept_commit (same acceptance, outputs and errors)
 * committing every layer: cache slot prefix_len[b] + d of layer l <- layer l's tree K/V
 * of path[d], for l = 0 .. n_layers-1.  Layer l's cache is at l * cache_layer_stride
 * elements and its tree K/V at l * tree_layer_stride elements (eagle_tree_verify_layers
 * writes them at total_nodes * Hkv * D).  All layers share `cache`'s strides and
 * capacity.  Strides must be positive multiples of 16 bytes when n_layers > 1, else
 * EAGLE_ERR_ARG.  A rejected sequence (accept_len -1) is committed in no layer. */
int eagle_accept_commit_layers(int32_t batch, const int32_t* tree_off, int32_t max_nodes, const int32_t* parent,
                               const int32_t* tokens, const int32_t* argmax, const uint64_t* anc,
                               int32_t mask_words, const int32_t* depth, const void* k_tree, const void* v_tree,
                               void* k_cache, void* v_cache, const eagle_cache_layout* cache, int32_t n_kv_heads,
                               int32_t head_dim, int32_t dtype, int32_t n_layers, int64_t cache_layer_stride,
                               int64_t tree_layer_stride, int32_t* prefix_len, const float* h_nodes,
                               int32_t hidden, float* next_feature, int32_t max_accept, int32_t* accept_len,
                               int32_t* path, int32_t* out_tokens, int32_t* next_token, int32_t* dev_status,
                               void* stream);

/* eagle_draft_kv_commit: after an acceptance call, the draft head's cache slots of the
 * committed positions recomputed from the target's true features.  The draft's cache is
 * indexed by the same positions as the target's: slot t holds the draft layer's K/V of
 * the row W_fc [f_(t-1) ; E[token_t]] at position t, f_(t-1) the target's feature at t - 1.
 * Per sequence b with L = accept_len[b] >= 0 and P = prefix_len[b] - L - 1 (prefix_len
 * already advanced by the commit), for d = 0..L:
 *   f = root_feature[b] (d = 0: the feature that preceded this step's root, as given to
 *       eagle_draft_expand) or h_nodes[tree_off[b] + path[b][d-1]] (d >= 1);
 *   row = W_fc [f ; embed[tokens[tree_off[b] + path[b][d]]]];
 *   slot P + d of dk_cache/dv_cache <- rotary(K rows of W_qkv RMSNorm(row)) at position
 *       P + d, and the V rows of W_qkv RMSNorm(row) (RMSNorm with draft_layer->ln_attn).
 * A sequence with accept_len -1 is left alone.  Inputs: w_fc [H][2H] and draft_layer
 * (ln_attn, w_qkv; layout as eagle_draft_expand), embed [V][H], tokens and h_nodes
 * [total_nodes][H] f32 of the verified trees, root_feature [B][H] f32 (must not be the
 * buffer the acceptance call wrote next_feature into), accept_len [B] and path
 * [B][max_accept + 1] from the acceptance call.  bf16 with head_dim 128 only
 * (EAGLE_ERR_UNSUPPORTED otherwise).  Device error: a slot >= capacity sets
 * *dev_status = EAGLE_ERR_CAPACITY and that row is not written.
 * Workspace: eagle_workspace_size(4, dims, batch, 0, max_accept + 1, 0, NULL). */
int eagle_draft_kv_commit(const eagle_dims* dims, const void* w_fc, const eagle_layer_w* draft_layer,
                          const void* embed, int32_t batch, const int32_t* tree_off, const int32_t* tokens,
                          const float* h_nodes, const float* root_feature, const int32_t* accept_len,
                          const int32_t* path, int32_t max_accept, const int32_t* prefix_len, void* dk_cache,
                          void* dv_cache, const eagle_cache_layout* cache, int32_t* dev_status, void* workspace,
                          size_t ws_bytes, void* stream);

/* ---- workspace -------------------------------------------------------------
 * Bytes of workspace a call needs.  which: 0 = eagle_tree_verify and
 * eagle_tree_verify_layers, 1 = eagle_draft_expand, 2 = eagle_fuse_features,
 * 3 = eagle_tree_verify_sample, 4 = eagle_draft_kv_commit (max_nodes = max_accept + 1).
 * params is used only for which == 1.  Returns 0 for unsupported arguments. */
size_t eagle_workspace_size(int32_t which, const eagle_dims* dims, int32_t batch, int32_t total_nodes,
                            int32_t max_nodes, int32_t max_prefix, const eagle_draft_params* params);

/* Zero-fill a workspace (once, after allocating it); enqueued on stream. */
int eagle_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* ---- per-kernel timing --------------------------------------------------------
 * A timer owns HIP events; calls given a timer record an event pair around each
 * kernel they launch, tagged by stage.  Stages: 0 tree_build, 1 qkv, 2 attention,
 * 3 attention_merge, 4 o_proj, 5 gate_up, 6 down, 7 lm_head, 8 accept_commit,
 * 9 draft_fc, 10 draft_topk, 11 draft_select, 12 other.  capacity = event pairs
 * recorded before the timer must be read. */
eagle_timer* eagle_timer_create(int32_t capacity);
void eagle_timer_destroy(eagle_timer* t);
/* Synchronises on the recorded events, adds elapsed ms per stage into
 * ms[EAGLE_N_STAGES] and launch counts into count[EAGLE_N_STAGES], and resets. */
int eagle_timer_collect(eagle_timer* t, double* ms, int32_t* count);
/* Record only the stages whose bit (1 << stage) is set in stage_mask (default: all).
 * Each recorded event pair separates two kernels on the stream, so timing every
 * stage slows the step down; timing one stage keeps the step close to untimed. */
int eagle_timer_select(eagle_timer* t, uint32_t stage_mask);
#define EAGLE_N_STAGES 13

const char* eagle_status_str(int status);
int eagle_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H_ */
