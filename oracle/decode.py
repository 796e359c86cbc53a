"""A stack of decoder layers under one LM head, tree verification through the stack, the
KV commit of every layer, the draft head's KV update from the target's true features, and
the two decode loops (plain greedy decoding and EAGLE steps) built from them.

TEST INFRASTRUCTURE (fp64 oracle; see the package docstring for who may import it).

Sources: "Speculative decoding with EAGLE" page, Deep dive and Technical insight (a draft
proposes, the target verifies every candidate in one pass and keeps the longest correct
prefix, so the emitted text is exactly what the target alone would produce; the draft
works on the target's hidden features and is fed the true embedding of the next token);
"LLM parallel decoding EAGLE" page, section on how EAGLE works (the draft head predicts
from the target's final hidden features; tree attention verifies all nodes at once);
"yuhuili" page (the draft reads the target's second-top-layer features).

Readings where the pages are silent:
  * the target is a stack of Llama-style layers (oracle.layer.layer_rows) applied in
    order, each with its own KV cache; the LM head (final RMSNorm, W_lm) follows the last
    layer; a node's feature is the last layer's output before the final norm;
  * every layer sees the same tree: the same ancestor mask and the same positions
    prefix_len + depth; committing a path writes each layer's tree K/V of the path into
    that layer's cache slots prefix_len .. prefix_len + L;
  * the draft's KV cache is indexed by the same positions as the target's.  Its slot t
    holds the draft layer's K/V of the row W_fc [f_{t-1} ; E[token_t]] at position t,
    where f_{t-1} is the target's feature at position t - 1.  After a step commits the
    path root .. leaf at slots P .. P + L, those slots of the draft cache are recomputed
    from true features: slot P from the step's root feature (the previous leaf's), slot
    P + d (d >= 1) from the target feature of path node d - 1 and the token of node d;
  * plain greedy decoding is verification of one-node trees: the root is the last token,
    its argmax is the next token, its K/V are committed.
"""
import numpy as np

from .accept import accept_sequence, commit_sequence
from .layer import as_f64, layer_rows, linear, lm_head_argmax, rms_norm, rope_rotate_half
from .tree import tree_encode


def verify_forward_layers(dims, weights, layers, x, parents, prefix_len, k_caches, v_caches, *,
                          embed_tokens=None, want_logits=False):
    """One verification pass of B trees through ``layers`` (a list of layer weight dicts).

    x [sum N][H] node inputs, or None with ``embed_tokens`` (x = embed[tokens]);
    k_caches/v_caches [n_layers][B][Hkv][cap][D]; prefix_len [B].
    Returns dict: k_tree, v_tree [n_layers][sum N][Hkv][D], h [sum N][H] (the last layer's
    output), argmax, maxlogit, gap, encs (and logits)."""
    if x is None:
        x = as_f64(weights["embed"][np.asarray(embed_tokens)])
    else:
        x = as_f64(x)
    nl = len(layers)
    Hkv, D = dims.n_kv_heads, dims.head_dim
    empty = np.zeros((0, Hkv, D))
    k_parts = [[] for _ in range(nl)]
    v_parts = [[] for _ in range(nl)]
    h_parts, encs = [], []
    r0 = 0
    for b, par in enumerate(parents):
        P = int(prefix_len[b])
        enc = tree_encode(par, P)
        encs.append(enc)
        hcur = x[r0:r0 + len(par)]
        for li, lw in enumerate(layers):
            res = layer_rows(dims, lw, hcur, enc.pos, as_f64(k_caches[li][b, :, :P]), as_f64(v_caches[li][b, :, :P]),
                             empty, empty, enc.anc)
            k_parts[li].append(res["k"])
            v_parts[li].append(res["v"])
            hcur = res["h"]
        h_parts.append(hcur)
        r0 += len(par)
    h = np.concatenate(h_parts)
    am, mx, gap, logits = lm_head_argmax(dims, weights, h)
    out = dict(k_tree=np.stack([np.concatenate(p) for p in k_parts]),
               v_tree=np.stack([np.concatenate(p) for p in v_parts]),
               h=h, argmax=am, maxlogit=mx, gap=gap, encs=encs)
    if want_logits:
        out["logits"] = logits
    return out


def commit_layers(k_caches, v_caches, b, k_tree, v_tree, node0, path, prefix_len):
    """Every layer's tree K/V of ``path`` (local node ids of the tree whose first node is
    row node0) into that layer's cache slots prefix_len ..; returns the new prefix length."""
    newP = prefix_len
    for li in range(len(k_caches)):
        newP = commit_sequence(k_caches[li][b], v_caches[li][b], k_tree[li][node0:], v_tree[li][node0:], path,
                               prefix_len)
    return newP


def draft_kv_rows(dims, dweights, embed, feats, tokens, pos):
    """K and V [n][Hkv][D] of the draft layer for the rows W_fc [feats ; E[tokens]] at
    positions pos: RMSNorm with the layer's attention gain, the K and V rows of W_qkv,
    rotary on K (the draft layer's own attention is not needed for its K/V)."""
    Hq, Hkv, D = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    n = len(tokens)
    rows = np.concatenate([as_f64(feats), as_f64(embed[np.asarray(tokens)])], axis=1) @ as_f64(dweights["w_fc"]).T
    xh = rms_norm(rows, dweights["ln_attn"], dims.rms_eps) if dims.rms_eps > 0 else rows
    qkv = linear(xh, dweights["w_qkv"])
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    if dims.rope_theta > 0:
        k = rope_rotate_half(k, pos, dims.rope_theta)
    return k, v


def draft_kv_commit(dims, dweights, embed, dk_cache_b, dv_cache_b, root_feature_b, h_tree, tokens_tree, path,
                    prefix_len_old):
    """The draft cache slots prefix_len_old + d, d = 0..L, of one sequence from the true
    features (see the module docstring); h_tree/tokens_tree are this tree's node features
    and tokens, path its accepted path root .. leaf.  Modifies the caches in place and
    returns the (K, V) rows written."""
    feats = [as_f64(root_feature_b)] + [h_tree[path[d - 1]] for d in range(1, len(path))]
    toks = [int(tokens_tree[p]) for p in path]
    pos = prefix_len_old + np.arange(len(path))
    k, v = draft_kv_rows(dims, dweights, embed, np.stack(feats), toks, pos)
    cap = dk_cache_b.shape[1]
    if prefix_len_old + len(path) > cap:
        raise ValueError("draft cache capacity exceeded")
    for d in range(len(path)):
        dk_cache_b[:, prefix_len_old + d] = k[d]
        dv_cache_b[:, prefix_len_old + d] = v[d]
    return k, v


def eagle_decode(dims, weights, layers, k_caches, v_caches, prefix_len, root_token, root_feature, trees, *,
                 draft=None):
    """EAGLE decode loop for one sequence (batch index 0 of the caches) over the given trees.

    trees: a list of (parent, tokens) pairs, one per step; the loop replaces each tree's
    root token by the current root (the previous step's bonus).  Each step verifies the
    tree through the stack, accepts the longest matching path, commits every layer's K/V
    and, with ``draft`` = (dweights, dk_cache, dv_cache), updates the draft cache from the
    true features.  The caches are modified in place.  Returns (emitted tokens, final
    prefix length, root token, root feature, per-step accept lengths)."""
    P = int(prefix_len)
    root, feat = int(root_token), as_f64(root_feature)
    emitted, lens = [], []
    for par, toks in trees:
        toks = [root] + [int(t) for t in toks[1:]]
        out = verify_forward_layers(dims, weights, layers, None, [par], [P], k_caches, v_caches,
                                    embed_tokens=toks)
        L, path, acc, nxt, leaf = accept_sequence(par, toks, out["argmax"], out["encs"][0].depth)
        newP = commit_layers(k_caches, v_caches, 0, out["k_tree"], out["v_tree"], 0, path, P)
        if draft is not None:
            dweights, dk, dv = draft
            draft_kv_commit(dims, dweights, weights["embed"], dk[0], dv[0], feat, out["h"], toks, path, P)
        emitted.extend(acc)
        lens.append(L)
        P, root, feat = newP, nxt, out["h"][leaf]
    return emitted, P, root, feat, lens


def greedy_decode(dims, weights, layers, k_caches, v_caches, prefix_len, root_token, n_tokens):
    """Plain greedy decoding of one sequence (batch index 0): each step verifies the
    one-node tree of the last token, commits its K/V in every layer and emits its argmax.
    Returns (tokens emitted, features h of the consumed tokens, top-2 gaps)."""
    P = int(prefix_len)
    t = int(root_token)
    toks, feats, gaps = [], [], []
    for _ in range(n_tokens):
        out = verify_forward_layers(dims, weights, layers, None, [[-1]], [P], k_caches, v_caches, embed_tokens=[t])
        P = commit_layers(k_caches, v_caches, 0, out["k_tree"], out["v_tree"], 0, [0], P)
        t = int(out["argmax"][0])
        toks.append(t)
        feats.append(out["h"][0])
        gaps.append(float(out["gap"][0]))
    return toks, feats, gaps
