"""Convenience runner for one verification step (tree encode -> verify -> accept + commit).

Allocates the per-step device buffers once for a maximum batch shape and calls the
three C entry points in order on the current stream.  Argument marshalling only;
all arithmetic runs in the HIP library.
"""
import torch

from . import _abi as A


LAYER_MATRICES = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "w_fc")


def with_packed_weights(weights, *, lm_head=True, layer=True):
    """A shallow copy of a weights dict with w_lm (lm_head) and the layer matrices present
    (layer: w_qkv, w_o, w_gate, w_up, w_down, w_fc) replaced by fragment-blocked copies
    written by eagle_pack_fragments; pass lm_layout=1 / weight_layout=1 to the runners with
    it.  A load-time step: each packed copy takes as much device memory as its source."""
    w = dict(weights)
    if lm_head and w.get("w_lm") is not None:
        w["w_lm"] = A.eagle_pack_fragments(weights["w_lm"])
    if layer:
        for k in LAYER_MATRICES:
            if w.get(k) is not None:
                w[k] = A.eagle_pack_fragments(weights[k])
    return w



class TreeVerifier:
    """lm_layout: 0 if weights["w_lm"] is row-major [vocab][hidden], 1 if fragment-blocked;
    weight_layout: the same for the layer matrices.  sample=True adds the buffers of
    verification and acceptance at temperature T > 0 (verify_sample, accept_sample)."""

    def __init__(self, dims, weights, k_cache, v_cache, *, batch, max_total_nodes, max_nodes, max_prefix,
                 max_accept=None, device="cuda", lm_layout=0, weight_layout=0, sample=False):
        self.dims = dims
        self.dstruct = A.dims_struct(dims, lm_layout)
        self.lstruct = A.layer_struct(weights, weight_layout)
        self.w = weights
        self.k_cache = k_cache
        self.v_cache = v_cache
        self.B = batch
        self.max_total = max_total_nodes
        self.max_nodes = max_nodes
        self.max_prefix = max_prefix
        self.mw = (max_nodes + 63) // 64
        self.max_accept = max_accept if max_accept is not None else max_nodes - 1
        dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        H, Hkv, D = dims.hidden, dims.n_kv_heads, dims.head_dim
        M = max_total_nodes
        z = lambda *s, dtype=torch.int32: torch.zeros(*s, dtype=dtype, device=device)  # noqa: E731
        self.anc = z(M, self.mw, dtype=torch.int64)
        self.depth = z(M)
        self.pos = z(M)
        self.k_tree = z(M, Hkv, D, dtype=dt)
        self.v_tree = z(M, Hkv, D, dtype=dt)
        self.h = z(M, H, dtype=torch.float32)
        self.argmax = z(M)
        self.maxlogit = z(M, dtype=torch.float32)
        self.accept_len = z(batch)
        self.path = z(batch, self.max_accept + 1)
        self.out_tokens = z(batch, self.max_accept + 1)
        self.next_token = z(batch)
        self.next_feature = z(batch, H, dtype=torch.float32)
        self.status = z(1)
        ws = A.eagle_workspace_size(0, dims, batch, M, max_nodes, max_prefix)
        if sample:
            ws3 = A.eagle_workspace_size(3, dims, batch, M, max_nodes, max_prefix)
            ws = max(ws, ws3) if ws and ws3 else 0
            self.child_logit = z(M, dtype=torch.float32)
            self.rest_lse = z(M, dtype=torch.float32)
            self.rest_token = z(M)
        if ws == 0:
            raise A.EagleError(A.EAGLE_ERR_UNSUPPORTED, "eagle_workspace_size")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        A.eagle_workspace_init(self.workspace)

    def encode(self, tree_off, parent, prefix_len, total_nodes):
        A.eagle_tree_build(tree_off, parent, prefix_len, self.mw, self.anc, self.depth, self.pos, self.status,
                           total_nodes=total_nodes, max_nodes=self.max_nodes)

    def verify(self, tree_off, tokens, prefix_len, total_nodes, x=None, embed=None, dbg_attn=None, dbg_logits=None,
               timer=None):
        w = self.w
        A.eagle_tree_verify(self.dstruct, self.lstruct, w.get("final_ln"), w["w_lm"], tree_off, x,
                            embed if embed is not None else w.get("embed") if x is None else None, tokens, self.anc,
                            self.mw, self.pos, prefix_len, self.k_cache, self.v_cache, self.k_tree, self.v_tree,
                            self.h, self.argmax, self.maxlogit, self.workspace, total_nodes=total_nodes,
                            max_nodes=self.max_nodes, max_prefix=self.max_prefix, dbg_attn=dbg_attn,
                            dbg_logits=dbg_logits, timer=timer)

    def accept(self, tree_off, parent, tokens, prefix_len):
        d = self.dims
        A.eagle_accept_commit(tree_off, parent, tokens, self.argmax, self.anc, self.mw, self.depth, self.k_tree,
                              self.v_tree, self.k_cache, self.v_cache, prefix_len, self.h, self.next_feature,
                              self.accept_len, self.path, self.out_tokens, self.next_token, self.status,
                              max_nodes=self.max_nodes, max_accept=self.max_accept, n_kv_heads=d.n_kv_heads,
                              head_dim=d.head_dim, dtype=A.EAGLE_BF16 if d.dtype == "bf16" else A.EAGLE_F32,
                              hidden=d.hidden)

    def step(self, tree_off, parent, tokens, prefix_len, total_nodes, x=None, timer=None):
        self.encode(tree_off, parent, prefix_len, total_nodes)
        self.verify(tree_off, tokens, prefix_len, total_nodes, x=x, timer=timer)
        self.accept(tree_off, parent, tokens, prefix_len)

    def verify_sample(self, tree_off, tokens, parent, prefix_len, total_nodes, temperature, gumbel, x=None,
                      timer=None):
        """gumbel: [batch][vocab] f32 noise, one row per tree."""
        w = self.w
        A.eagle_tree_verify_sample(self.dstruct, self.lstruct, w.get("final_ln"), w["w_lm"], tree_off, x,
                                   w.get("embed") if x is None else None, tokens, parent, self.anc, self.mw,
                                   self.pos, prefix_len, self.k_cache, self.v_cache, temperature, gumbel,
                                   self.k_tree, self.v_tree, self.h, self.child_logit, self.rest_lse,
                                   self.rest_token, self.workspace, total_nodes=total_nodes,
                                   max_nodes=self.max_nodes, max_prefix=self.max_prefix, timer=timer)

    def accept_sample(self, tree_off, parent, tokens, u, prefix_len):
        """u: [total_nodes] f32 acceptance uniforms."""
        d = self.dims
        A.eagle_accept_commit_sample(tree_off, parent, tokens, self.child_logit, self.rest_lse, self.rest_token, u,
                                     self.k_tree, self.v_tree, self.k_cache, self.v_cache, prefix_len, self.h,
                                     self.next_feature, self.accept_len, self.path, self.out_tokens,
                                     self.next_token, self.status, max_nodes=self.max_nodes,
                                     max_accept=self.max_accept, n_kv_heads=d.n_kv_heads, head_dim=d.head_dim,
                                     dtype=A.EAGLE_BF16 if d.dtype == "bf16" else A.EAGLE_F32, hidden=d.hidden)

    def step_sample(self, tree_off, parent, tokens, prefix_len, total_nodes, temperature, gumbel, u, x=None,
                    timer=None):
        self.encode(tree_off, parent, prefix_len, total_nodes)
        self.verify_sample(tree_off, tokens, parent, prefix_len, total_nodes, temperature, gumbel, x=x, timer=timer)
        self.accept_sample(tree_off, parent, tokens, u, prefix_len)


class TreeDrafter:
    """Draft-tree expansion for a batch of sequences (eagle_draft_expand), with its
    output buffers and workspace allocated once.

    weights: the target's tensors (final_ln, w_lm, embed); draft_weights: w_fc and the
    draft decoder layer.  Trees come out compacted (tree_off, parent, tokens, cum) in
    arrays of batch * max_nodes entries, padded past tree_off[batch].  lm_layout: the
    layout of weights["w_lm"] (0 row-major, 1 fragment-blocked); weight_layout: the same
    for the draft matrices (w_fc and the draft layer)."""

    def __init__(self, dims, params, weights, draft_weights, dk_cache, dv_cache, *, batch, max_prefix,
                 device="cuda", lm_layout=0, weight_layout=0):
        self.dims = dims
        self.params = A.draft_params_struct(params)
        self.dstruct = A.dims_struct(dims, lm_layout)
        self.lstruct = A.layer_struct(draft_weights, weight_layout)
        self.w = weights
        self.dw = draft_weights
        self.dk_cache = dk_cache
        self.dv_cache = dv_cache
        self.B = batch
        self.max_prefix = max_prefix
        p = self.params
        self.max_nodes = p.max_nodes
        self.pool_cap = 1 + p.top_k + (p.depth - 1) * p.frontier * p.top_k
        N = batch * p.max_nodes
        z = lambda *s, dtype=torch.int32: torch.zeros(*s, dtype=dtype, device=device)  # noqa: E731
        self.tree_off = z(batch + 1)
        self.parent = z(N)
        self.tokens = z(N)
        self.cum = z(N, dtype=torch.float32)
        ws = A.eagle_workspace_size(1, dims, batch, 0, 0, max_prefix, self.params)
        if ws == 0:
            raise A.EagleError(A.EAGLE_ERR_UNSUPPORTED, "eagle_workspace_size")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        A.eagle_workspace_init(self.workspace)

    def expand(self, root_feature, root_token, prefix_len, timer=None):
        w, dw = self.w, self.dw
        A.eagle_draft_expand(self.dstruct, self.params, dw["w_fc"], self.lstruct, w["final_ln"], w["w_lm"],
                             w["embed"], root_feature, root_token, self.dk_cache, self.dv_cache, prefix_len,
                             self.tree_off, self.parent, self.tokens, self.cum, self.workspace,
                             max_prefix=self.max_prefix, timer=timer)

    def pool(self):
        """Candidate pool of the last expansion (device tensors)."""
        p, B, P = self.params, self.B, self.pool_cap
        dev = self.workspace.device
        out = dict(pool_n=torch.zeros(B, dtype=torch.int32, device=dev),
                   token=torch.zeros(B, P, dtype=torch.int32, device=dev),
                   parent=torch.zeros(B, P, dtype=torch.int32, device=dev),
                   depth=torch.zeros(B, P, dtype=torch.int32, device=dev),
                   cum=torch.zeros(B, P, dtype=torch.float32, device=dev),
                   logp=torch.zeros(B, P, dtype=torch.float32, device=dev),
                   expanded=torch.zeros(B, p.depth, p.frontier, dtype=torch.int32, device=dev))
        A.eagle_draft_pool(self.dstruct, self.params, B, self.max_prefix, self.workspace, out["pool_n"], out["token"],
                           out["parent"], out["depth"], out["cum"], out["logp"], out["expanded"])
        return out


class EagleStep:
    """One full speculative step on device, with no host synchronisation: draft a tree
    per sequence, encode it, verify every node with the target layer (inputs are the
    token embeddings), accept the longest matching path and commit its K/V.  The next
    step's roots are the accepted bonus tokens and their features."""

    def __init__(self, dims, params, weights, draft_weights, k_cache, v_cache, dk_cache, dv_cache, *, batch,
                 max_prefix, device="cuda", lm_layout=0, weight_layout=0, sample=False):
        self.drafter = TreeDrafter(dims, params, weights, draft_weights, dk_cache, dv_cache, batch=batch,
                                   max_prefix=max_prefix, device=device, lm_layout=lm_layout,
                                   weight_layout=weight_layout)
        M = self.drafter.max_nodes
        self.total = batch * M
        self.verifier = TreeVerifier(dims, weights, k_cache, v_cache, batch=batch, max_total_nodes=self.total,
                                     max_nodes=M, max_prefix=max_prefix, device=device, lm_layout=lm_layout,
                                     weight_layout=weight_layout, sample=sample)

    def step(self, root_feature, root_token, prefix_len, timer=None):
        d, v = self.drafter, self.verifier
        d.expand(root_feature, root_token, prefix_len, timer=timer)
        v.encode(d.tree_off, d.parent, prefix_len, self.total)
        v.verify(d.tree_off, d.tokens, prefix_len, self.total, timer=timer)
        v.accept(d.tree_off, d.parent, d.tokens, prefix_len)
        return v.next_feature, v.next_token

    def step_sample(self, root_feature, root_token, prefix_len, temperature, gumbel, u, timer=None):
        """The same step with acceptance at temperature T > 0 (needs sample=True): gumbel
        [batch][vocab] noise rows, u [batch * max_nodes] acceptance uniforms."""
        d, v = self.drafter, self.verifier
        d.expand(root_feature, root_token, prefix_len, timer=timer)
        v.encode(d.tree_off, d.parent, prefix_len, self.total)
        v.verify_sample(d.tree_off, d.tokens, d.parent, prefix_len, self.total, temperature, gumbel, timer=timer)
        v.accept_sample(d.tree_off, d.parent, d.tokens, u, prefix_len)
        return v.next_feature, v.next_token


class StackVerifier(TreeVerifier):
    """TreeVerifier through a stack of decoder layers (eagle_tree_verify_layers and
    eagle_accept_commit_layers).  weights: final_ln, w_lm (and embed); layers: one weight
    dict per layer (layout weight_layout); k_caches/v_caches [n_layers][B][Hkv][cap][D].
    k_tree/v_tree are [n_layers][max_total_nodes][Hkv][D]."""

    def __init__(self, dims, weights, layers, k_caches, v_caches, *, batch, max_total_nodes, max_nodes, max_prefix,
                 max_accept=None, device="cuda", lm_layout=0, weight_layout=0):
        super().__init__(dims, weights, k_caches[0], v_caches[0], batch=batch, max_total_nodes=max_total_nodes,
                         max_nodes=max_nodes, max_prefix=max_prefix, max_accept=max_accept, device=device,
                         lm_layout=lm_layout, weight_layout=weight_layout)
        self.layers = layers
        self.larr = A.layers_array(layers, weight_layout)
        self.n_layers = len(layers)
        self.k_caches = k_caches
        self.v_caches = v_caches
        n = self.n_layers
        self.k_tree = torch.zeros(n, *self.k_tree.shape, dtype=self.k_tree.dtype, device=device)
        self.v_tree = torch.zeros(n, *self.v_tree.shape, dtype=self.v_tree.dtype, device=device)

    def verify(self, tree_off, tokens, prefix_len, total_nodes, x=None, embed=None, dbg_attn=None, dbg_logits=None,
               timer=None):
        w = self.w
        A.eagle_tree_verify_layers(self.dstruct, self.larr, w.get("final_ln"), w["w_lm"], tree_off, x,
                                   embed if embed is not None else w.get("embed") if x is None else None, tokens,
                                   self.anc, self.mw, self.pos, prefix_len, self.k_caches, self.v_caches, self.k_tree,
                                   self.v_tree, self.h, self.argmax, self.maxlogit, self.workspace,
                                   total_nodes=total_nodes, max_nodes=self.max_nodes, max_prefix=self.max_prefix,
                                   dbg_attn=dbg_attn, dbg_logits=dbg_logits, timer=timer)

    def accept(self, tree_off, parent, tokens, prefix_len):
        d = self.dims
        A.eagle_accept_commit_layers(tree_off, parent, tokens, self.argmax, self.anc, self.mw, self.depth, self.k_tree,
                                     self.v_tree, self.k_caches, self.v_caches, prefix_len, self.h, self.next_feature,
                                     self.accept_len, self.path, self.out_tokens, self.next_token, self.status,
                                     max_nodes=self.max_nodes, max_accept=self.max_accept, n_kv_heads=d.n_kv_heads,
                                     head_dim=d.head_dim, dtype=A.EAGLE_BF16 if d.dtype == "bf16" else A.EAGLE_F32,
                                     hidden=d.hidden)


class DraftKV:
    """The draft-KV update after acceptance (eagle_draft_kv_commit) with its workspace."""

    def __init__(self, dims, weights, draft_weights, dk_cache, dv_cache, *, batch, max_accept, device="cuda",
                 weight_layout=0):
        self.dstruct = A.dims_struct(dims)
        self.lstruct = A.layer_struct(draft_weights, weight_layout)
        self.w = weights
        self.dw = draft_weights
        self.dk_cache = dk_cache
        self.dv_cache = dv_cache
        self.max_accept = max_accept
        ws = A.eagle_workspace_size(4, dims, batch, 0, max_accept + 1, 0)
        if ws == 0:
            raise A.EagleError(A.EAGLE_ERR_UNSUPPORTED, "eagle_workspace_size")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        A.eagle_workspace_init(self.workspace)

    def commit(self, verifier, tree_off, tokens, root_feature, prefix_len):
        """Slots of the path verifier.accept just committed, from verifier.h and root_feature
        (the feature given to this step's draft; not verifier.next_feature)."""
        v = verifier
        A.eagle_draft_kv_commit(self.dstruct, self.dw["w_fc"], self.lstruct, self.w["embed"], tree_off, tokens, v.h,
                                root_feature, v.accept_len, v.path, prefix_len, self.dk_cache, self.dv_cache,
                                self.workspace, v.status, max_accept=v.max_accept)


class EagleStackStep:
    """The full speculative step with a target of several layers: draft a tree per sequence,
    encode it, verify it through every layer, accept, commit every layer's K/V, then rewrite
    the draft cache slots of the committed path from the target's true features.  No host
    synchronisation.  step() returns (next_feature, next_token); the feature buffers
    alternate between two tensors, so the returned feature can be passed straight back as the
    next step's root feature."""

    def __init__(self, dims, params, weights, layers, draft_weights, k_caches, v_caches, dk_cache, dv_cache, *, batch,
                 max_prefix, device="cuda", lm_layout=0, weight_layout=0):
        self.drafter = TreeDrafter(dims, params, weights, draft_weights, dk_cache, dv_cache, batch=batch,
                                   max_prefix=max_prefix, device=device, lm_layout=lm_layout,
                                   weight_layout=weight_layout)
        M = self.drafter.max_nodes
        self.total = batch * M
        # an accepted path is at most the draft depth long
        self.verifier = StackVerifier(dims, weights, layers, k_caches, v_caches, batch=batch,
                                      max_total_nodes=self.total, max_nodes=M, max_prefix=max_prefix,
                                      max_accept=params.depth, device=device, lm_layout=lm_layout,
                                      weight_layout=weight_layout)
        self.dkv = DraftKV(dims, weights, draft_weights, dk_cache, dv_cache, batch=batch, max_accept=params.depth,
                           device=device, weight_layout=weight_layout)
        self.feats = [self.verifier.next_feature, torch.zeros_like(self.verifier.next_feature)]
        self.n = 0

    def step(self, root_feature, root_token, prefix_len, timer=None):
        d, v = self.drafter, self.verifier
        v.next_feature = self.feats[self.n % 2]
        if v.next_feature.data_ptr() == root_feature.data_ptr():
            v.next_feature = self.feats[(self.n + 1) % 2]
        self.n += 1
        d.expand(root_feature, root_token, prefix_len, timer=timer)
        v.encode(d.tree_off, d.parent, prefix_len, self.total)
        v.verify(d.tree_off, d.tokens, prefix_len, self.total, timer=timer)
        v.accept(d.tree_off, d.parent, d.tokens, prefix_len)
        self.dkv.commit(v, d.tree_off, d.tokens, root_feature, prefix_len)
        return v.next_feature, v.next_token


class GreedyStackDecoder:
    """Plain greedy decoding of a batch through the same layer stack and kernels: each step
    verifies the one-node tree of every sequence's last token, commits its K/V in every layer
    and emits its argmax.  step() returns the emitted tokens (device, [batch]), which are also
    the next step's inputs."""

    def __init__(self, dims, weights, layers, k_caches, v_caches, *, batch, max_prefix, device="cuda", lm_layout=0,
                 weight_layout=0):
        self.v = StackVerifier(dims, weights, layers, k_caches, v_caches, batch=batch, max_total_nodes=batch,
                               max_nodes=1, max_prefix=max_prefix, max_accept=0, device=device, lm_layout=lm_layout,
                               weight_layout=weight_layout)
        self.B = batch
        self.tree_off = torch.arange(batch + 1, dtype=torch.int32, device=device)
        self.parent = torch.full((batch,), -1, dtype=torch.int32, device=device)
        self.tokens = torch.zeros(batch, dtype=torch.int32, device=device)

    def step(self, tokens, prefix_len, timer=None):
        v = self.v
        self.tokens.copy_(tokens)
        v.encode(self.tree_off, self.parent, prefix_len, self.B)
        v.verify(self.tree_off, self.tokens, prefix_len, self.B, timer=timer)
        v.accept(self.tree_off, self.parent, self.tokens, prefix_len)
        return v.next_token


class PagePool:
    """Host-side page allocator of a paged KV cache, for continuous batching: sequences join
    and grow (pages taken from a free list), leave (pages returned for reuse), and each step
    runs on the block table of whichever sequences are active.  Page ids only: the pages
    themselves are caller-owned tensors [n_pages][Hkv][page_size][D] (or with a leading layer
    dimension), wrapped with paged()."""

    def __init__(self, n_pages, page_size, max_blocks, device="cuda"):
        self.n_pages = n_pages
        self.page_size = page_size
        self.max_blocks = max_blocks
        self.device = device
        self.free = list(range(n_pages))
        self.owned = {}

    def reserve(self, seq, n_tokens):
        """Pages for sequence ``seq`` so that it can hold n_tokens slots; returns its page list."""
        pages = self.owned.setdefault(seq, [])
        need = -(-n_tokens // self.page_size)
        if need > self.max_blocks:
            raise A.EagleError(A.EAGLE_ERR_CAPACITY, f"PagePool: {n_tokens} tokens exceed max_blocks")
        while len(pages) < need:
            if not self.free:
                raise A.EagleError(A.EAGLE_ERR_CAPACITY, "PagePool: out of pages")
            pages.append(self.free.pop(0))
        return pages

    def release(self, seq):
        """Return a sequence's pages; they are the next ones handed out."""
        self.free[:0] = self.owned.pop(seq, [])

    def table(self, seqs):
        """Device block table [len(seqs)][max_blocks] of the given sequences (-1: unowned)."""
        t = torch.full((len(seqs), self.max_blocks), -1, dtype=torch.int32)
        for i, q in enumerate(seqs):
            pg = self.owned.get(q, [])
            t[i, :len(pg)] = torch.tensor(pg, dtype=torch.int32)
        return t.to(self.device)

    def paged(self, pages, table):
        return A.PagedCache(pages, table, self.page_size)
