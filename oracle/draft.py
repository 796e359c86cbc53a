"""Draft-head tree expansion (EAGLE feature-level drafting, EAGLE-2-style dynamic trees).

TEST INFRASTRUCTURE (fp64 oracle; see the package docstring for who may import it).

Sources: "Speculative decoding with EAGLE" page, Deep dive / Technical insight
(the head predicts the next hidden feature, is fed the true embedding of the
previous token alongside the feature, and reuses the target's LM head);
"LLM parallel decoding EAGLE" page, section on how EAGLE works (a one-layer
decoder head; several token candidates per predicted feature, each expanded
further into a tree), its EAGLE vs EAGLE-2 table (confidence-based adaptive
trees that give more nodes to confident paths and prune unconfident ones
early), and FAQ Q3 (confidence threshold 0.3; a lower threshold widens the
search); "yuhuili" author page (the draft's confidence stands in for the
acceptance rate).

Readings where the pages leave steps open, level-synchronous:
  1. a node's draft row is W_fc [f_parent ; E[token]] (feature first, no
     bias); the root's f_parent is the given feature.  The row runs through
     the one draft decoder layer at position prefix_len + depth, attending to
     the draft KV prefix and to the draft-tree nodes on its own root path;
     its output is the predicted feature f_hat;
  2. draft logits are the target's LM head on RMSNorm(f_hat) (final norm
     included); log-probabilities are the log-softmax over the whole
     vocabulary; the top_k tokens (ties: lower id) become children;
  3. cum(child) = cum(parent) + min(0, log p); cum(root) = 0;
  4. a child is expandable iff its own probability p >= conf_threshold;
  5. the next frontier is the ``frontier`` best expandable children of this
     level by (cum desc, depth asc, generation order asc), where generation
     order is (level, rank of the parent in its frontier, child rank);
     frontier 0 means no limit;
  6. after ``depth`` levels (or an empty frontier) the tree is the root plus
     the best max_nodes - 1 generated nodes by the same key; cum never grows
     along a path, so the kept set is ancestor-closed; nodes are re-indexed by
     (depth asc, cum desc, generation order asc).
"""
import numpy as np

from .layer import as_f64, layer_rows, lm_head_logits


def fuse_features(w_fuse, low, mid, high):
    """EAGLE-3 draft input: the root feature is a fusion of the target's low-, mid- and
    high-level features instead of its top feature ("LLM parallel decoding EAGLE" page,
    EAGLE vs EAGLE-2 table and FAQ; "yuhuili" page, EAGLE-3).  The pages give no formula;
    reading: one linear map without bias, W_fuse [H][3H] applied to [f_low; f_mid; f_high]
    in that order.  Returns [B][H] in fp64; the draft expansion then takes it as the root
    feature unchanged."""
    x = np.concatenate([as_f64(low), as_f64(mid), as_f64(high)], axis=-1)
    return x @ as_f64(w_fuse).T


def log_softmax(z):
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))


def topk_stable(row, k):
    """Indices of the k largest entries, ties to the lower index."""
    return np.argsort(-row, kind="stable")[:k]


def _key(node):
    return (-node["cum"], node["depth"], node["gen"])


def draft_select_level(children, frontier, tau):
    """Step 4-5: indices (into ``children``) of the next frontier, in rank order."""
    idx = [i for i, c in enumerate(children) if c["p"] >= tau]
    idx.sort(key=lambda i: _key(children[i]))
    return idx if frontier <= 0 else idx[:frontier]


def draft_rerank(pool, max_nodes):
    """Step 6: returns (parent, tokens, cum, kept pool ids) of the final tree."""
    rest = sorted(range(1, len(pool)), key=lambda i: _key(pool[i]))[: max_nodes - 1]
    kept = set(rest) | {0}
    for i in rest:
        assert pool[i]["parent"] in kept
    order = [0] + sorted(rest, key=lambda i: (pool[i]["depth"], -pool[i]["cum"], pool[i]["gen"]))
    new = {old: k for k, old in enumerate(order)}
    parent = [-1] + [new[pool[i]["parent"]] for i in order[1:]]
    tokens = [int(pool[i]["token"]) for i in order]
    cum = [float(pool[i]["cum"]) for i in order]
    return parent, tokens, cum, order


def draft_expand(dims, params, weights, dweights, root_feature, root_token, dk_cache, dv_cache, prefix_len,
                 *, trace=False, force=None):
    """Expand one draft tree per sequence.  Returns a list of per-sequence dicts
    (parent, tokens, cum, and with ``trace`` the pool and per-level records).

    ``force`` (teacher forcing, for checking another implementation's decisions):
    a per-sequence list of dicts with ``tokens[level]`` = the children tokens of
    each expanded row and ``frontier[level]`` = the pool ids expanded on that
    level (level >= 2).  The oracle then takes those decisions instead of its own
    top-k and selection; every value (features, log-probabilities, cum) is still
    its own, and the trace records its own top-k and selection beside them."""
    H, Hkv, D = dims.hidden, dims.n_kv_heads, dims.head_dim
    E = weights["embed"]
    out = []
    for b in range(len(root_token)):
        P = int(prefix_len[b])
        k_pre = as_f64(dk_cache[b, :, :P])
        v_pre = as_f64(dv_cache[b, :, :P])
        pool = [dict(token=int(root_token[b]), parent=-1, depth=0, cum=0.0, gen=(0, 0, 0), p=1.0)]
        proc_of = {}             # pool id -> index among processed nodes
        proc_anc = []            # per processed node: set of processed indices on its root path
        proc_k = np.zeros((0, Hkv, D))
        proc_v = np.zeros((0, Hkv, D))
        fhat = {}
        frontier = [0]
        levels = []
        for level in range(1, params.depth + 1):
            if not frontier:
                break
            m0 = len(proc_anc)
            x = np.empty((len(frontier), 2 * H))
            for r, n in enumerate(frontier):
                par = pool[n]["parent"]
                f_par = as_f64(root_feature[b]) if par < 0 else fhat[par]
                x[r, :H] = f_par
                x[r, H:] = as_f64(E[pool[n]["token"]])
            rows = x @ as_f64(dweights["w_fc"]).T
            pos = np.array([P + pool[n]["depth"] for n in frontier])
            vis = np.zeros((len(frontier), m0 + len(frontier)), dtype=bool)
            for r, n in enumerate(frontier):
                par = pool[n]["parent"]
                anc = set() if par < 0 else set(proc_anc[proc_of[par]])
                anc.add(m0 + r)
                proc_of[n] = m0 + r
                proc_anc.append(anc)
                vis[r, sorted(anc)] = True
            res = layer_rows(dims, dweights, rows, pos, k_pre, v_pre, proc_k, proc_v, vis)
            proc_k = np.concatenate([proc_k, res["k"]])
            proc_v = np.concatenate([proc_v, res["v"]])
            z = lm_head_logits(dims, weights, res["h"])
            logp = log_softmax(z)
            fb = force[b] if force is not None else None
            children = []
            tops = []
            own_tops = []
            for r, n in enumerate(frontier):
                fhat[n] = res["h"][r]
                own = topk_stable(logp[r], params.top_k + 1)
                own_tops.append((own, logp[r][own]))
                top = own[: params.top_k] if fb is None else np.asarray(fb["tokens"][level][r])
                tops.append(top)
                for c, t in enumerate(top):
                    children.append(dict(token=int(t), parent=n, depth=pool[n]["depth"] + 1,
                                         cum=pool[n]["cum"] + min(0.0, float(logp[r, t])),
                                         gen=(level, r, c), p=float(np.exp(logp[r, t])), logp=float(logp[r, t])))
            base = len(pool)
            pool.extend(children)
            sel = draft_select_level(children, params.frontier, params.conf_threshold)
            nxt = [base + i for i in sel]
            if trace:
                levels.append(dict(frontier=list(frontier), rows=rows, fhat=res["h"],
                                   logp_top=[lp[t] for lp, t in zip(logp, tops)], tops=tops, own_tops=own_tops,
                                   zscale=np.abs(z).max(axis=1),
                                   children=list(range(base, len(pool))), next=nxt))
            if fb is not None:
                nxt = list(fb["frontier"].get(level + 1, []))
            frontier = nxt
        parent, tokens, cum, order = draft_rerank(pool, params.max_nodes)
        rec = dict(parent=parent, tokens=tokens, cum=cum)
        if trace:
            rec.update(pool=pool, levels=levels, order=order)
        out.append(rec)
    return out
