"""Target forward pass over a token tree, in float64.

TEST INFRASTRUCTURE (fp64 oracle; see the package docstring for who may import it).

Sources: "LLM parallel decoding EAGLE" page, section on how EAGLE works (tree
attention: all nodes verified in one forward pass, each node seeing the
prefix and its own ancestors); "Speculative decoding with EAGLE" page,
Technical insight (the target's LM head turns features into tokens; accepted
tokens must equal the target's argmax choice).

Readings where the pages are silent (the layer is a Llama-style pre-norm
decoder layer, as the workload shapes say):
  * RMSNorm x / sqrt(mean(x^2) + eps) * gain, no biases, SiLU-gated MLP;
  * rotary embedding in the rotate-half pairing (j, j + D/2) with inverse
    frequency theta^(-2j/D), applied to q and k at position prefix_len + depth;
    cached prefix keys are taken as already rotated;
  * softmax scale 1/sqrt(D); a node attends to every prefix key and to the
    tree keys of its ancestors and itself; KV head of query head h is h // g;
  * the attention-only layer (no norms) is y = x + W_o o and logits = W_lm y;
  * argmax is the first index of the maximum.
Weights are [out][in]; bf16 inputs are widened exactly to float64.
"""
import numpy as np

from workloads.bf16 import bf16_bits_to_f64

_ROW_CHUNK = 4096


def as_f64(a):
    """Exact float64 view of a bf16-bit (uint16) or float32/float64 array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def linear(x, w):
    """x @ w.T with w [out][in] widened to float64 one row-chunk at a time."""
    n_out = w.shape[0]
    out = np.empty((x.shape[0], n_out), dtype=np.float64)
    for r in range(0, n_out, _ROW_CHUNK):
        out[:, r:r + _ROW_CHUNK] = x @ as_f64(w[r:r + _ROW_CHUNK]).T
    return out


def rms_norm(x, gain, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * as_f64(gain)


def silu(z):
    return z / (1.0 + np.exp(-z))


def rope_rotate_half(x, pos, theta):
    """x [n][heads][D] rotated at positions pos [n]: pairs (j, j + D/2), angle pos * theta^(-2j/D)."""
    D = x.shape[-1]
    half = D // 2
    inv_freq = theta ** (-(2.0 * np.arange(half)) / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attend(q, k_pre, v_pre, k_nodes, v_nodes, vis):
    """Tree-masked GQA attention.

    q [n][Hq][D]; k_pre, v_pre [Hkv][P][D] (every row sees every prefix key);
    k_nodes, v_nodes [m][Hkv][D]; vis [n][m] bool (row r sees node key j iff vis[r, j]).
    Returns o [n][Hq][D] = sum_j softmax_j(q.k_j / sqrt(D)) v_j over the visible keys.
    """
    n, Hq, D = q.shape
    Hkv = k_pre.shape[0]
    g = Hq // Hkv
    P = k_pre.shape[1]
    o = np.empty_like(q)
    visible = np.concatenate([np.ones((n, P), dtype=bool), vis], axis=1)
    for kvh in range(Hkv):
        K = np.concatenate([k_pre[kvh], k_nodes[:, kvh]], axis=0)  # [P+m][D]
        V = np.concatenate([v_pre[kvh], v_nodes[:, kvh]], axis=0)
        for h in range(kvh * g, (kvh + 1) * g):
            s = (q[:, h] @ K.T) / np.sqrt(D)
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[:, h] = p @ V
    return o


def layer_rows(dims, w, x, pos, k_pre, v_pre, k_prev, v_prev, vis):
    """One decoder layer over ``n`` new rows of a tree.

    x [n][H] (float64); pos [n]; k_pre/v_pre [Hkv][P][D] the cached prefix;
    k_prev/v_prev [m0][Hkv][D] tree nodes already processed (may be empty);
    vis [n][m0 + n]: which earlier tree nodes and which of the new rows each row sees.
    Returns dict with q, k, v (new rows, post-rotary), attn [n][Hq*D], y, h [n][H].
    """
    H, D, Hq, Hkv = dims.hidden, dims.head_dim, dims.n_q_heads, dims.n_kv_heads
    n = x.shape[0]
    norm = dims.rms_eps > 0
    xh = rms_norm(x, w["ln_attn"], dims.rms_eps) if norm else x
    qkv = linear(xh, w["w_qkv"])
    q = qkv[:, : Hq * D].reshape(n, Hq, D)
    k = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(n, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    if dims.rope_theta > 0:
        q = rope_rotate_half(q, pos, dims.rope_theta)
        k = rope_rotate_half(k, pos, dims.rope_theta)
    k_all = np.concatenate([k_prev, k], axis=0)
    v_all = np.concatenate([v_prev, v], axis=0)
    o = attend(q, k_pre, v_pre, k_all, v_all, vis).reshape(n, Hq * D)
    y = x + linear(o, w["w_o"])
    if dims.ffn > 0:
        yh = rms_norm(y, w["ln_mlp"], dims.rms_eps)
        a = silu(linear(yh, w["w_gate"])) * linear(yh, w["w_up"])
        h = y + linear(a, w["w_down"])
    else:
        h = y
    return dict(q=q, k=k, v=v, attn=o, y=y, h=h)


def lm_head_logits(dims, weights, h, rows=None):
    """logits = W_lm RMSNorm(h) (attention-only layer: W_lm h); [n][V] float64."""
    hn = rms_norm(h, weights["final_ln"], dims.rms_eps) if dims.rms_eps > 0 else h
    if rows is not None:
        hn = hn[rows]
    return linear(hn, weights["w_lm"])


def lm_head_argmax(dims, weights, h):
    """Per row: first index of the maximum logit, the maximum, and the top-2 gap."""
    logits = lm_head_logits(dims, weights, h)
    am = np.argmax(logits, axis=1)
    mx = logits[np.arange(len(am)), am]
    tmp = logits.copy()
    tmp[np.arange(len(am)), am] = -np.inf
    gap = mx - tmp.max(axis=1)
    return am.astype(np.int64), mx, gap, logits


def verify_forward(dims, weights, x, parents, prefix_len, k_cache, v_cache, *, embed_tokens=None,
                   want_logits=True):
    """One verification pass over B trees (their nodes concatenated).

    x [sum N][H] node inputs, or None with ``embed_tokens`` (then x = embed[tokens]).
    k_cache/v_cache [B][Hkv][cap][D]; prefix_len [B].
    Returns dict: q, k_tree, v_tree, attn, y, h, argmax, maxlogit, gap, (logits), encs.
    """
    from .tree import tree_encode
    if x is None:
        tokens = embed_tokens
        x = as_f64(weights["embed"][np.asarray(tokens)])
    else:
        x = as_f64(x)
    sizes = [len(p) for p in parents]
    off = np.concatenate([[0], np.cumsum(sizes)])
    parts = []
    encs = []
    for b, par in enumerate(parents):
        P = int(prefix_len[b])
        enc = tree_encode(par, P)
        encs.append(enc)
        r0, r1 = off[b], off[b + 1]
        Dh = dims.head_dim
        empty = np.zeros((0, dims.n_kv_heads, Dh))
        res = layer_rows(dims, weights, x[r0:r1], enc.pos,
                         as_f64(k_cache[b, :, :P]), as_f64(v_cache[b, :, :P]), empty, empty, enc.anc)
        parts.append(res)
    out = {key: np.concatenate([p[key] for p in parts]) for key in ("q", "k", "v", "attn", "y", "h")}
    out["k_tree"] = out.pop("k")
    out["v_tree"] = out.pop("v")
    am, mx, gap, logits = lm_head_argmax(dims, weights, out["h"])
    out.update(argmax=am, maxlogit=mx, gap=gap, encs=encs)
    if want_logits:
        out["logits"] = logits
    return out
