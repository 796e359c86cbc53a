"""The five synthetic workloads, seeded and random-init.

Shapes follow the benchmark configurations of this project (a tiny fp32
attention layer; Llama-3-8B- and 70B-shaped single decoder layers in bf16;
ragged dynamic trees; the full draft+verify step).  Values: N(0, s) means
standard deviation s; weights N(0, 0.02), KV prefix and node hidden states
N(0, 1), token ids uniform.  RMSNorm gains are 1 unless a test asks for
random gains.  MLP widths 14336 / 28672 are the public Llama-3 widths (the
pages give none).

Every tensor has its own stream ``numpy.random.default_rng([seed, tensor_id,
chunk])``; big tensors are drawn in row chunks on a thread pool, so a draw is
reproducible regardless of thread count.  bf16 tensors are drawn in float32
and rounded once (RNE) to bf16 bit patterns (uint16).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

from .bf16 import f32_to_bf16_bits
from . import trees as T


@dataclass(frozen=True)
class LayerDims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int            # 0: attention-only layer (no norms, no MLP)
    vocab: int
    rope_theta: float   # 0: no rotary embedding
    rms_eps: float      # 0: no RMSNorm anywhere
    dtype: str          # "bf16" or "f32"

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads


@dataclass(frozen=True)
class DraftParams:
    depth: int = 6          # expansion levels
    top_k: int = 10         # children per expanded node
    frontier: int = 10      # nodes expanded per level (0: unbounded)
    max_nodes: int = 60     # final tree size, root included
    conf_threshold: float = 0.0  # a child is expandable iff its own probability >= this


LLAMA8B = LayerDims(4096, 32, 8, 128, 14336, 128256, 5.0e5, 1e-5, "bf16")
LLAMA70B = LayerDims(8192, 64, 8, 128, 28672, 128256, 5.0e5, 1e-5, "bf16")
TINY = LayerDims(256, 4, 4, 64, 0, 1000, 0.0, 0.0, "f32")

CONFIGS = {
    1: dict(name="tiny-fp32-attn-26node", dims=TINY, batch=1, prefix=128, tree="static26"),
    2: dict(name="llama3-8b-layer-60node-P2048", dims=LLAMA8B, batch=1, prefix=2048, tree="static60"),
    3: dict(name="llama3-8b-layer-B4-dynamic40to120-P4096", dims=LLAMA8B, batch=4, prefix=4096,
            tree="dynamic"),
    4: dict(name="llama3-70b-layer-60node-P32768", dims=LLAMA70B, batch=1, prefix=32768, tree="static60"),
    5: dict(name="llama3-8b-eagle-step-B16-P2048", dims=LLAMA8B, batch=16, prefix=2048, tree="draft",
            draft=DraftParams()),
}

# tensor ids of the per-tensor random streams
TID = dict(x=1, k_prefix=2, v_prefix=3, tokens=4, w_qkv=10, w_o=11, w_gate=12, w_up=13, w_down=14,
           w_lm=15, embed=16, w_fc=17, ln_attn=18, ln_mlp=19, final_ln=20,
           d_w_qkv=30, d_w_o=31, d_w_gate=32, d_w_up=33, d_w_down=34, d_ln_attn=35, d_ln_mlp=36,
           d_k_prefix=37, d_v_prefix=38, root_feature=39, root_token=40, tree=41, w_fuse=42, fuse_feats=43, gumbel=44, accept_u=45)

_ROWS_PER_CHUNK = 2048


def _pool_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_tensor(seed, tid, shape, std, dtype):
    """N(0, std) tensor, float32 or bf16 bits, drawn in row chunks."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, inner), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def work(c):
        r0 = c * _ROWS_PER_CHUNK
        r1 = min(rows, r0 + _ROWS_PER_CHUNK)
        rng = np.random.default_rng([seed, tid, c])
        a = rng.standard_normal((r1 - r0, inner), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(a) if dtype == "bf16" else a

    n_chunks = (rows + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK
    if n_chunks <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        with ThreadPoolExecutor(_pool_workers()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out.reshape(shape)


def gain_vector(seed, tid, n, std, dtype):
    """RMSNorm gain: ones, or 1 + N(0, std) when a test asks for random gains."""
    g = np.ones(n, dtype=np.float32)
    if std > 0:
        g += np.random.default_rng([seed, tid, 0]).standard_normal(n, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(g) if dtype == "bf16" else g


def layer_weights(seed, dims: LayerDims, prefix="", gamma_std=0.0, tid_offset=0):
    """Random-init decoder-layer weights, [out][in] row-major.  tid_offset shifts every
    tensor id (layer l of a stack uses LAYER_TID_STRIDE * l)."""
    H, D, Hq, Hkv, F = dims.hidden, dims.head_dim, dims.n_q_heads, dims.n_kv_heads, dims.ffn
    t = dims.dtype
    tid = lambda name: TID[prefix + name] + tid_offset  # noqa: E731
    w = {
        "w_qkv": normal_tensor(seed, tid("w_qkv"), (dims.qkv_rows, H), 0.02, t),
        "w_o": normal_tensor(seed, tid("w_o"), (H, Hq * D), 0.02, t),
    }
    if F > 0:
        w["ln_attn"] = gain_vector(seed, tid("ln_attn"), H, gamma_std, t)
        w["ln_mlp"] = gain_vector(seed, tid("ln_mlp"), H, gamma_std, t)
        w["w_gate"] = normal_tensor(seed, tid("w_gate"), (F, H), 0.02, t)
        w["w_up"] = normal_tensor(seed, tid("w_up"), (F, H), 0.02, t)
        w["w_down"] = normal_tensor(seed, tid("w_down"), (H, F), 0.02, t)
    return w


@dataclass
class Workload:
    cfg_id: int
    name: str
    seed: int
    dims: LayerDims
    batch: int
    prefix_len: np.ndarray          # [B] int32
    cache_cap: int
    parents: list                   # B parent arrays (None when the draft builds the trees)
    tree_off: Optional[np.ndarray]  # [B+1] int32
    tokens: Optional[np.ndarray]    # [sum N] int32, root token first in each tree
    x: Optional[np.ndarray]         # [sum N][H] node hidden states (None: x = embed[tokens])
    weights: dict                   # layer weights + final_ln, w_lm, (embed)
    k_cache: np.ndarray             # [B][Hkv][cap][D], prefix filled, rest zero
    v_cache: np.ndarray
    draft: Optional[DraftParams] = None
    draft_weights: dict = field(default_factory=dict)  # w_fc, layer weights of the draft head
    dk_cache: Optional[np.ndarray] = None
    dv_cache: Optional[np.ndarray] = None
    root_feature: Optional[np.ndarray] = None  # [B][H] float32
    root_token: Optional[np.ndarray] = None    # [B] int32

    @property
    def n_nodes(self):
        return int(self.tree_off[-1]) if self.tree_off is not None else 0

    @property
    def mask_words(self):
        nmax = max(len(p) for p in self.parents)
        return (nmax + 63) // 64


def mini_dims(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1408, vocab=5003,
              rope_theta=5.0e5, rms_eps=1e-5, dtype="bf16"):
    """Reduced shapes for parity tests the oracle finishes in seconds (still several tiles, ragged tails)."""
    return LayerDims(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rope_theta, rms_eps, dtype)


def _kv_cache(seed, tid, B, Hkv, cap, D, prefix_len, dtype):
    P = int(max(prefix_len)) if len(prefix_len) else 0
    full = np.zeros((B, Hkv, cap, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    if P > 0:
        drawn = normal_tensor(seed, tid, (B * Hkv * P, D), 1.0, dtype).reshape(B, Hkv, P, D)
        for b in range(B):
            full[b, :, : prefix_len[b]] = drawn[b, :, : prefix_len[b]]
    return full


def make_workload(cfg_id, seed=None, *, dims: LayerDims = None, batch=None, prefix=None,
                  parents=None, gamma_std=0.0, cache_slack=16, draft: DraftParams = None):
    """Build the seeded workload of configuration ``cfg_id`` (optionally with overrides)."""
    base = CONFIGS[cfg_id]
    seed = 1000 + cfg_id if seed is None else seed
    dims = dims or base["dims"]
    B = batch or base["batch"]
    P = base["prefix"] if prefix is None else prefix
    prefix_len = np.array(P if np.ndim(P) else [P] * B, dtype=np.int32)
    assert prefix_len.shape == (B,)
    t = dims.dtype
    H, D, Hkv, V = dims.hidden, dims.head_dim, dims.n_kv_heads, dims.vocab
    tok_rng = np.random.default_rng([seed, TID["tokens"]])

    kind = base["tree"]
    if parents is None:
        if kind == "static26":
            parents = [T.static_tree_26() for _ in range(B)]
        elif kind == "static60":
            parents = [T.static_tree_60() for _ in range(B)]
        elif kind == "dynamic":
            parents = [T.eagle2_style_tree(seed, b)[0] for b in range(B)]
        elif kind == "draft":
            parents = None
    draft = draft if draft is not None else base.get("draft")

    weights = layer_weights(seed, dims, gamma_std=gamma_std)
    if dims.rms_eps > 0:
        weights["final_ln"] = gain_vector(seed, TID["final_ln"], H, gamma_std, t)
    weights["w_lm"] = normal_tensor(seed, TID["w_lm"], (V, H), 0.02, t)

    max_depth = 16 if parents is None else max(max(T.depths(p)) for p in parents)
    if draft is not None:
        max_depth = max(max_depth, draft.depth)
    cap = int(prefix_len.max()) + max_depth + 1 + cache_slack
    k_cache = _kv_cache(seed, TID["k_prefix"], B, Hkv, cap, D, prefix_len, t)
    v_cache = _kv_cache(seed, TID["v_prefix"], B, Hkv, cap, D, prefix_len, t)

    wl = Workload(cfg_id=cfg_id, name=base["name"], seed=seed, dims=dims, batch=B,
                  prefix_len=prefix_len, cache_cap=cap, parents=parents, tree_off=None, tokens=None,
                  x=None, weights=weights, k_cache=k_cache, v_cache=v_cache, draft=draft)
    if parents is not None:
        sizes = [len(p) for p in parents]
        wl.tree_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        wl.tokens = np.concatenate([T.tree_tokens(tok_rng, p, V) for p in parents]).astype(np.int32)
        if kind != "draft":
            wl.x = normal_tensor(seed, TID["x"], (int(wl.tree_off[-1]), H), 1.0, t)
    if draft is not None or kind == "draft":
        weights["embed"] = normal_tensor(seed, TID["embed"], (V, H), 0.02, t)
        dw = layer_weights(seed, dims, prefix="d_", gamma_std=gamma_std)
        dw["w_fc"] = normal_tensor(seed, TID["w_fc"], (H, 2 * H), 0.02, t)
        wl.draft_weights = dw
        wl.dk_cache = _kv_cache(seed, TID["d_k_prefix"], B, Hkv, cap, D, prefix_len, t)
        wl.dv_cache = _kv_cache(seed, TID["d_v_prefix"], B, Hkv, cap, D, prefix_len, t)
        wl.root_feature = normal_tensor(seed, TID["root_feature"], (B, H), 1.0, "f32")
        wl.root_token = np.random.default_rng([seed, TID["root_token"]]).integers(0, V, size=B).astype(np.int32)
    return wl


def eagle3_inputs(wl: Workload):
    """Seeded EAGLE-3 draft inputs for a draft workload: the fusion matrix W_fuse [H][3H]
    (N(0, 0.02)) and each sequence's low-, mid- and high-level target features [B][3H]
    (N(0, 1)), both stored as bf16 bits."""
    H, B = wl.dims.hidden, wl.batch
    w_fuse = normal_tensor(wl.seed, TID["w_fuse"], (H, 3 * H), 0.02, "bf16")
    feats = normal_tensor(wl.seed, TID["fuse_feats"], (B, 3 * H), 1.0, "bf16")
    return w_fuse, feats


def sample_inputs(wl: Workload, draw=0, n_nodes=None):
    """Seeded random inputs of acceptance at temperature T > 0 for a workload with trees:
    one row of standard Gumbel noise per tree, gumbel [B][V] = -log(-log U) with U uniform
    on the open interval (0, 1) (float64, stored as float32), and one acceptance uniform per
    node, u [sum N] in [0, 1) (float32).  ``draw`` selects an independent set; ``n_nodes``
    overrides sum N (e.g. batch * max_nodes for trees a draft step will build)."""
    B, V = wl.batch, wl.dims.vocab
    n = wl.n_nodes if n_nodes is None else int(n_nodes)
    rng = np.random.default_rng([wl.seed, TID["gumbel"], draw])
    U = rng.random((B, V))
    U = np.where(U > 0.0, U, np.nextafter(0.0, 1.0))
    gumbel = (-np.log(-np.log(U))).astype(np.float32)
    u = np.random.default_rng([wl.seed, TID["accept_u"], draw]).random(n).astype(np.float32)
    return gumbel, u


def with_trees(wl: Workload, parents, tokens=None, x_seed_tid=None):
    """Replace the trees of a workload (e.g. with trees built by a draft step)."""
    sizes = [len(p) for p in parents]
    wl2 = replace(wl, parents=[list(p) for p in parents])
    wl2.tree_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    if tokens is None:
        rng = np.random.default_rng([wl.seed, TID["tokens"], 7])
        tokens = np.concatenate([T.tree_tokens(rng, p, wl.dims.vocab) for p in parents])
    wl2.tokens = np.asarray(tokens, dtype=np.int32)
    if wl.x is not None or x_seed_tid is not None:
        wl2.x = normal_tensor(wl.seed, x_seed_tid or TID["x"], (int(wl2.tree_off[-1]), wl.dims.hidden), 1.0,
                              wl.dims.dtype)
    return wl2


LAYER_TID_STRIDE = 1000  # tensor ids of layer l of a stack: TID[...] + LAYER_TID_STRIDE * l


@dataclass
class StackWorkload:
    """A target of n_layers decoder layers under one LM head, with one KV cache per layer,
    and a draft head (w_fc + one layer) with its own cache, for decode loops."""
    seed: int
    dims: LayerDims
    n_layers: int
    batch: int
    prefix_len: np.ndarray   # [B] int32
    cache_cap: int
    layers: list             # n_layers weight dicts (w_qkv, w_o, ln_attn, ln_mlp, w_gate, w_up, w_down)
    weights: dict            # final_ln, w_lm, embed
    k_caches: np.ndarray     # [n_layers][B][Hkv][cap][D], prefix filled, rest zero
    v_caches: np.ndarray
    draft_weights: dict      # w_fc and the draft layer
    dk_cache: np.ndarray     # [B][Hkv][cap][D]
    dv_cache: np.ndarray
    root_feature: np.ndarray  # [B][H] float32: the feature that precedes each root token
    root_token: np.ndarray    # [B] int32


def stack_workload(seed, dims: LayerDims, n_layers, *, batch=1, prefix=64, cache_cap=None, gamma_std=0.0,
                   embed_std=0.02, lm_std=0.02):
    """Seeded stack of n_layers random-init layers (layer 0 draws the same tensors as the
    single-layer workloads of this seed), prefix K/V N(0, 1) per layer, embedding
    N(0, embed_std), LM head N(0, lm_std), a draft head, root features N(0, 1) and uniform
    root tokens."""
    B = batch
    prefix_len = np.array(prefix if np.ndim(prefix) else [prefix] * B, dtype=np.int32)
    H, D, Hkv, V, t = dims.hidden, dims.head_dim, dims.n_kv_heads, dims.vocab, dims.dtype
    cap = cache_cap or int(prefix_len.max()) + 64
    layers = [layer_weights(seed, dims, gamma_std=gamma_std, tid_offset=LAYER_TID_STRIDE * l) for l in range(n_layers)]
    weights = dict(w_lm=normal_tensor(seed, TID["w_lm"], (V, H), lm_std, t),
                   embed=normal_tensor(seed, TID["embed"], (V, H), embed_std, t))
    if dims.rms_eps > 0:
        weights["final_ln"] = gain_vector(seed, TID["final_ln"], H, gamma_std, t)
    kc = np.stack([_kv_cache(seed, TID["k_prefix"] + LAYER_TID_STRIDE * l, B, Hkv, cap, D, prefix_len, t)
                   for l in range(n_layers)])
    vc = np.stack([_kv_cache(seed, TID["v_prefix"] + LAYER_TID_STRIDE * l, B, Hkv, cap, D, prefix_len, t)
                   for l in range(n_layers)])
    dw = layer_weights(seed, dims, prefix="d_", gamma_std=gamma_std)
    dw["w_fc"] = normal_tensor(seed, TID["w_fc"], (H, 2 * H), 0.02, t)
    return StackWorkload(
        seed=seed, dims=dims, n_layers=n_layers, batch=B, prefix_len=prefix_len, cache_cap=cap, layers=layers,
        weights=weights, k_caches=kc, v_caches=vc, draft_weights=dw,
        dk_cache=_kv_cache(seed, TID["d_k_prefix"], B, Hkv, cap, D, prefix_len, t),
        dv_cache=_kv_cache(seed, TID["d_v_prefix"], B, Hkv, cap, D, prefix_len, t),
        root_feature=normal_tensor(seed, TID["root_feature"], (B, H), 1.0, "f32"),
        root_token=np.random.default_rng([seed, TID["root_token"]]).integers(0, V, size=B).astype(np.int32))
