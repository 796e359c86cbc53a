"""ctypes binding of libeagle_hip.so: the C ABI declared in include/eagle.h.

Argument marshalling only.  Every function takes torch tensors (device memory) or
Python ints, passes raw pointers and sizes to the library, and raises EagleError
when the library returns a non-OK status.  All work is enqueued on the current
torch stream (or the stream given) and nothing is synchronised.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeagle_hip.so")

EAGLE_OK = 0
EAGLE_ERR_ARG = -1
EAGLE_ERR_TREE = -2
EAGLE_ERR_CAPACITY = -3
EAGLE_ERR_UNSUPPORTED = -4
EAGLE_ERR_HIP = -5
EAGLE_ERR_WORKSPACE = -6
EAGLE_BF16 = 0
EAGLE_F32 = 1
N_STAGES = 13
STAGES = ["tree_build", "qkv", "attention", "attention_merge", "o_proj", "gate_up", "down", "lm_head",
          "accept_commit", "draft_fc", "draft_topk", "draft_select", "other"]


class EagleError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class EagleDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("lm_layout", ctypes.c_int32)]


class EagleLayerW(ctypes.Structure):
    _fields_ = [("ln_attn", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("ln_mlp", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("layout", ctypes.c_int32)]


class EagleCacheLayout(ctypes.Structure):
    _fields_ = [("batch_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("capacity", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


class PagedCache:
    """A paged KV cache, accepted wherever a cache tensor is: pages [n_pages][Hkv][page_size][D]
    (or [n_layers][n_pages][Hkv][page_size][D] for a stack of layers) addressed through
    block_table [B][max_blocks] (device int32 page ids).  Sequence b's token t lives in page
    block_table[b][t // page_size] at slot t % page_size; capacity = max_blocks * page_size."""

    def __init__(self, pages, block_table, page_size):
        self.pages = pages
        self.block_table = block_table
        self.page_size = int(page_size)
        if pages.shape[-2] != self.page_size:
            raise EagleError(EAGLE_ERR_ARG, "PagedCache: pages must be [..][n_pages][Hkv][page_size][D]")

    @property
    def shape(self):
        return self.pages.shape

    def stride(self, i):
        return self.pages.stride(i)

    def data_ptr(self):
        return self.pages.data_ptr()

    def __getitem__(self, layer):
        return PagedCache(self.pages[layer], self.block_table, self.page_size)


class EagleDraftParams(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32), ("top_k", ctypes.c_int32), ("frontier", ctypes.c_int32),
                ("max_nodes", ctypes.c_int32), ("conf_threshold", ctypes.c_float)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t

# name -> (restype, argtypes), exactly the prototypes of include/eagle.h
PROTOTYPES = {
    "eagle_tree_build": (_I, [_I, _P, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
    "eagle_tree_verify": (_I, [ctypes.POINTER(EagleDims), ctypes.POINTER(EagleLayerW), _P, _P, _I, _P, _I, _I,
                               _P, _P, _P, _P, _I, _P, _P, _I, _P, _P, ctypes.POINTER(EagleCacheLayout), _P, _P,
                               _P, _P, _P, _P, _P, _P, _S, _P, _P]),
    "eagle_tree_verify_noalloc": (_I, [ctypes.POINTER(EagleDims), ctypes.POINTER(EagleLayerW), _P, _P, _I, _P, _I,
                                       _I, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P,
                                       ctypes.POINTER(EagleCacheLayout), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "eagle_accept_commit": (_I, [_I, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                 ctypes.POINTER(EagleCacheLayout), _I, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P,
                                 _P, _P]),
    "eagle_tree_verify_sample": (_I, [ctypes.POINTER(EagleDims), ctypes.POINTER(EagleLayerW), _P, _P, _I, _P, _I,
                                      _I, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P,
                                      ctypes.POINTER(EagleCacheLayout), ctypes.c_float, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _S, _P, _P]),
    "eagle_accept_commit_sample": (_I, [_I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.POINTER(EagleCacheLayout), _I, _I, _I, _P, _P, _I, _P, _I, _P, _P,
                                        _P, _P, _P, _P]),
    "eagle_tree_verify_layers": (_I, [ctypes.POINTER(EagleDims), _I, ctypes.POINTER(EagleLayerW), _P, _P, _I, _P,
                                      _I, _I, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P,
                                      ctypes.POINTER(EagleCacheLayout), ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _S, _P, _P]),
    "eagle_accept_commit_layers": (_I, [_I, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                        ctypes.POINTER(EagleCacheLayout), _I, _I, _I, _I, ctypes.c_int64,
                                        ctypes.c_int64, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P]),
    "eagle_draft_kv_commit": (_I, [ctypes.POINTER(EagleDims), _P, ctypes.POINTER(EagleLayerW), _P, _I, _P, _P, _P,
                                   _P, _P, _P, _I, _P, _P, _P, ctypes.POINTER(EagleCacheLayout), _P, _P, _S, _P]),
    "eagle_draft_expand": (_I, [ctypes.POINTER(EagleDims), ctypes.POINTER(EagleDraftParams), _P,
                                ctypes.POINTER(EagleLayerW), _P, _P, _P, _I, _P, _P, _P, _P,
                                ctypes.POINTER(EagleCacheLayout), _P, _I, _P, _P, _P, _P, _P, _S, _P, _P]),
    "eagle_draft_pool": (_I, [ctypes.POINTER(EagleDims), ctypes.POINTER(EagleDraftParams), _I, _I, _P, _S, _P, _P,
                              _P, _P, _P, _P, _P, _P]),
    "eagle_workspace_size": (_S, [_I, ctypes.POINTER(EagleDims), _I, _I, _I, _I, ctypes.POINTER(EagleDraftParams)]),
    "eagle_workspace_init": (_I, [_P, _S, _P]),
    "eagle_pack_fragments": (_I, [_P, _I, _I, _P, _P]),
    "eagle_fuse_features": (_I, [ctypes.POINTER(EagleDims), _P, _I, _P, _I, _P, _P, _S, _P]),
    "eagle_timer_create": (_P, [_I]),
    "eagle_timer_destroy": (None, [_P]),
    "eagle_timer_collect": (_I, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
    "eagle_timer_select": (_I, [_P, ctypes.c_uint32]),
    "eagle_status_str": (ctypes.c_char_p, [_I]),
    "eagle_abi_version": (_I, []),
}


def lib():
    """Load the in-tree library (built by __graft_entry__.build()); fails loudly if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(st):
    return lib().eagle_status_str(int(st)).decode()


def _check(st, where):
    if st != EAGLE_OK:
        raise EagleError(st, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _t(timer):
    return None if timer is None else ctypes.c_void_p(timer.handle)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dims_struct(dims, lm_layout=0):
    """EagleDims from a workloads.LayerDims-like object; lm_layout 1: w_lm is fragment-blocked."""
    return EagleDims(dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                     float(dims.rope_theta), float(dims.rms_eps), EAGLE_BF16 if dims.dtype == "bf16" else EAGLE_F32,
                     int(lm_layout))


def layer_struct(w, layout=0):
    """EagleLayerW from a dict of device tensors (missing entries -> NULL); layout 1: the
    matrices are fragment-blocked (eagle_pack_fragments)."""
    g = lambda k: w[k].data_ptr() if w.get(k) is not None else None  # noqa: E731
    return EagleLayerW(g("ln_attn"), g("w_qkv"), g("w_o"), g("ln_mlp"), g("w_gate"), g("w_up"), g("w_down"),
                       int(layout))


def cache_struct(cache):
    """EagleCacheLayout of a contiguous [B][Hkv][cap][D] tensor or of a PagedCache."""
    if isinstance(cache, PagedCache):
        n_pages, Hkv, ps, D = cache.pages.shape
        s = cache.pages.stride()
        maxb = cache.block_table.shape[1]
        return EagleCacheLayout(s[0], s[1], s[2], maxb * ps, cache.block_table.data_ptr(), ps, maxb, n_pages)
    B, Hkv, cap, D = cache.shape
    s = cache.stride()
    return EagleCacheLayout(s[0], s[1], s[2], cap, None, 0, 0, 0)


def draft_params_struct(p):
    """EagleDraftParams from any object with depth, top_k, frontier, max_nodes, conf_threshold."""
    if isinstance(p, EagleDraftParams):
        return p
    return EagleDraftParams(int(p.depth), int(p.top_k), int(p.frontier), int(p.max_nodes), float(p.conf_threshold))


def eagle_tree_build(tree_off, parent, prefix_len, mask_words, anc, depth, pos, dev_status=None, *,
                     total_nodes, max_nodes, stream=None):
    B = tree_off.numel() - 1
    st = lib().eagle_tree_build(B, _p(tree_off), total_nodes, max_nodes, _p(parent), _p(prefix_len), mask_words,
                                _p(anc), _p(depth), _p(pos), _p(dev_status), _stream(stream))
    _check(st, "eagle_tree_build")


def eagle_tree_verify(dims, layer, final_ln, w_lm, tree_off, x_in, embed, tokens, anc, mask_words, pos, prefix_len,
                      k_cache, v_cache, k_tree, v_tree, h_out, argmax, maxlogit, workspace, *, total_nodes,
                      max_nodes, max_prefix, dbg_attn=None, dbg_logits=None, timer=None, stream=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    lw = layer_struct(layer) if not isinstance(layer, EagleLayerW) else layer
    cl = cache_struct(k_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_tree_verify(ctypes.byref(d), ctypes.byref(lw), _p(final_ln), _p(w_lm), B, _p(tree_off),
                                 total_nodes, max_nodes, _p(x_in), _p(embed), _p(tokens), _p(anc), mask_words,
                                 _p(pos), _p(prefix_len), max_prefix, _p(k_cache), _p(v_cache), ctypes.byref(cl),
                                 _p(k_tree), _p(v_tree), _p(h_out), _p(argmax), _p(maxlogit), _p(dbg_attn),
                                 _p(dbg_logits), _p(workspace), workspace.numel() * workspace.element_size(),
                                 _t(timer), _stream(stream))
    _check(st, "eagle_tree_verify")


NOALLOC_MAX_BYTES = 32 << 20  # EAGLE_NOALLOC_MAX_BYTES


def eagle_tree_verify_noalloc(dims, layer, final_ln, w_lm, tree_off, x_in, embed, tokens, anc, mask_words, pos,
                              prefix_len, k_cache, v_cache, k_tree, v_tree, h_out, argmax, maxlogit, *, total_nodes,
                              max_nodes, max_prefix, dbg_attn=None, dbg_logits=None, timer=None, stream=None):
    """eagle_tree_verify without a workspace: the library's own per-GPU scratch is used."""
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    lw = layer_struct(layer) if not isinstance(layer, EagleLayerW) else layer
    cl = cache_struct(k_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_tree_verify_noalloc(ctypes.byref(d), ctypes.byref(lw), _p(final_ln), _p(w_lm), B, _p(tree_off),
                                         total_nodes, max_nodes, _p(x_in), _p(embed), _p(tokens), _p(anc),
                                         mask_words, _p(pos), _p(prefix_len), max_prefix, _p(k_cache), _p(v_cache),
                                         ctypes.byref(cl), _p(k_tree), _p(v_tree), _p(h_out), _p(argmax),
                                         _p(maxlogit), _p(dbg_attn), _p(dbg_logits), _t(timer), _stream(stream))
    _check(st, "eagle_tree_verify_noalloc")


def layers_array(layers, layout=0):
    """A ctypes array of EagleLayerW, one per layer dict (or EagleLayerW) of ``layers``."""
    structs = [lw if isinstance(lw, EagleLayerW) else layer_struct(lw, layout) for lw in layers]
    return (EagleLayerW * len(structs))(*structs)


def eagle_tree_verify_layers(dims, layers, final_ln, w_lm, tree_off, x_in, embed, tokens, anc, mask_words, pos,
                             prefix_len, k_caches, v_caches, k_tree, v_tree, h_out, argmax, maxlogit, workspace, *,
                             total_nodes, max_nodes, max_prefix, dbg_attn=None, dbg_logits=None, timer=None,
                             stream=None):
    """layers: a ctypes array from layers_array (or a list of layer dicts); k_caches/v_caches
    [n_layers][B][Hkv][cap][D]; k_tree/v_tree [n_layers][total_nodes][Hkv][D]."""
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    arr = layers if isinstance(layers, ctypes.Array) else layers_array(layers)
    cl = cache_struct(k_caches[0])
    if k_caches.stride(0) != v_caches.stride(0):
        raise EagleError(EAGLE_ERR_ARG, "eagle_tree_verify_layers: K and V caches differ in layout")
    B = tree_off.numel() - 1
    st = lib().eagle_tree_verify_layers(ctypes.byref(d), len(arr), arr, _p(final_ln), _p(w_lm), B, _p(tree_off),
                                        total_nodes, max_nodes, _p(x_in), _p(embed), _p(tokens), _p(anc),
                                        mask_words, _p(pos), _p(prefix_len), max_prefix, _p(k_caches),
                                        _p(v_caches), ctypes.byref(cl), k_caches.stride(0), _p(k_tree), _p(v_tree),
                                        _p(h_out), _p(argmax), _p(maxlogit), _p(dbg_attn), _p(dbg_logits),
                                        _p(workspace), workspace.numel() * workspace.element_size(), _t(timer),
                                        _stream(stream))
    _check(st, "eagle_tree_verify_layers")


def eagle_accept_commit_layers(tree_off, parent, tokens, argmax, anc, mask_words, depth, k_tree, v_tree, k_caches,
                               v_caches, prefix_len, h_nodes, next_feature, accept_len, path, out_tokens, next_token,
                               dev_status=None, *, max_nodes, max_accept, n_kv_heads, head_dim, dtype, hidden,
                               stream=None):
    """k_caches/v_caches [n_layers][B][Hkv][cap][D]; k_tree/v_tree [n_layers][total_nodes][Hkv][D]."""
    cl = cache_struct(k_caches[0])
    B = tree_off.numel() - 1
    nl = k_caches.shape[0]
    if k_caches.stride(0) != v_caches.stride(0) or k_tree.stride(0) != v_tree.stride(0) or k_tree.shape[0] != nl:
        raise EagleError(EAGLE_ERR_ARG, "eagle_accept_commit_layers: layer layouts differ")
    st = lib().eagle_accept_commit_layers(B, _p(tree_off), max_nodes, _p(parent), _p(tokens), _p(argmax), _p(anc),
                                          mask_words, _p(depth), _p(k_tree), _p(v_tree), _p(k_caches),
                                          _p(v_caches), ctypes.byref(cl), n_kv_heads, head_dim, dtype, nl,
                                          k_caches.stride(0), k_tree.stride(0), _p(prefix_len), _p(h_nodes), hidden,
                                          _p(next_feature), max_accept, _p(accept_len), _p(path), _p(out_tokens),
                                          _p(next_token), _p(dev_status), _stream(stream))
    _check(st, "eagle_accept_commit_layers")


def eagle_draft_kv_commit(dims, w_fc, draft_layer, embed, tree_off, tokens, h_nodes, root_feature, accept_len, path,
                          prefix_len, dk_cache, dv_cache, workspace, dev_status=None, *, max_accept, stream=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    lw = layer_struct(draft_layer) if not isinstance(draft_layer, EagleLayerW) else draft_layer
    cl = cache_struct(dk_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_draft_kv_commit(ctypes.byref(d), _p(w_fc), ctypes.byref(lw), _p(embed), B, _p(tree_off),
                                     _p(tokens), _p(h_nodes), _p(root_feature), _p(accept_len), _p(path),
                                     max_accept, _p(prefix_len), _p(dk_cache), _p(dv_cache), ctypes.byref(cl),
                                     _p(dev_status), _p(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check(st, "eagle_draft_kv_commit")


def eagle_accept_commit(tree_off, parent, tokens, argmax, anc, mask_words, depth, k_tree, v_tree, k_cache, v_cache,
                        prefix_len, h_nodes, next_feature, accept_len, path, out_tokens, next_token, dev_status=None,
                        *, max_nodes, max_accept, n_kv_heads, head_dim, dtype, hidden, stream=None):
    cl = cache_struct(k_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_accept_commit(B, _p(tree_off), max_nodes, _p(parent), _p(tokens), _p(argmax), _p(anc),
                                   mask_words, _p(depth), _p(k_tree), _p(v_tree), _p(k_cache), _p(v_cache),
                                   ctypes.byref(cl), n_kv_heads, head_dim, dtype, _p(prefix_len), _p(h_nodes),
                                   hidden, _p(next_feature), max_accept, _p(accept_len), _p(path), _p(out_tokens),
                                   _p(next_token), _p(dev_status), _stream(stream))
    _check(st, "eagle_accept_commit")


def eagle_tree_verify_sample(dims, layer, final_ln, w_lm, tree_off, x_in, embed, tokens, parent, anc, mask_words,
                             pos, prefix_len, k_cache, v_cache, temperature, gumbel, k_tree, v_tree, h_out,
                             child_logit, rest_lse, rest_token, workspace, *, total_nodes, max_nodes, max_prefix,
                             timer=None, stream=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    lw = layer_struct(layer) if not isinstance(layer, EagleLayerW) else layer
    cl = cache_struct(k_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_tree_verify_sample(ctypes.byref(d), ctypes.byref(lw), _p(final_ln), _p(w_lm), B, _p(tree_off),
                                        total_nodes, max_nodes, _p(x_in), _p(embed), _p(tokens), _p(parent),
                                        _p(anc), mask_words, _p(pos), _p(prefix_len), max_prefix, _p(k_cache),
                                        _p(v_cache), ctypes.byref(cl), float(temperature), _p(gumbel), _p(k_tree),
                                        _p(v_tree), _p(h_out), _p(child_logit), _p(rest_lse), _p(rest_token),
                                        _p(workspace), workspace.numel() * workspace.element_size(), _t(timer),
                                        _stream(stream))
    _check(st, "eagle_tree_verify_sample")


def eagle_accept_commit_sample(tree_off, parent, tokens, child_logit, rest_lse, rest_token, u, k_tree, v_tree,
                               k_cache, v_cache, prefix_len, h_nodes, next_feature, accept_len, path, out_tokens,
                               next_token, dev_status=None, *, max_nodes, max_accept, n_kv_heads, head_dim, dtype,
                               hidden, stream=None):
    cl = cache_struct(k_cache)
    B = tree_off.numel() - 1
    st = lib().eagle_accept_commit_sample(B, _p(tree_off), max_nodes, _p(parent), _p(tokens), _p(child_logit),
                                          _p(rest_lse), _p(rest_token), _p(u), _p(k_tree), _p(v_tree), _p(k_cache),
                                          _p(v_cache), ctypes.byref(cl), n_kv_heads, head_dim, dtype, _p(prefix_len),
                                          _p(h_nodes), hidden, _p(next_feature), max_accept, _p(accept_len),
                                          _p(path), _p(out_tokens), _p(next_token), _p(dev_status), _stream(stream))
    _check(st, "eagle_accept_commit_sample")


def eagle_draft_expand(dims, params, w_fc, draft_layer, final_ln, w_lm, embed, root_feature, root_token, dk_cache,
                       dv_cache, prefix_len, tree_off, parent, tokens, cum_logp, workspace, *, max_prefix,
                       timer=None, stream=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    lw = layer_struct(draft_layer) if not isinstance(draft_layer, EagleLayerW) else draft_layer
    cl = cache_struct(dk_cache)
    B = root_token.numel()
    params = draft_params_struct(params)
    st = lib().eagle_draft_expand(ctypes.byref(d), ctypes.byref(params), _p(w_fc), ctypes.byref(lw), _p(final_ln),
                                  _p(w_lm), _p(embed), B, _p(root_feature), _p(root_token), _p(dk_cache),
                                  _p(dv_cache), ctypes.byref(cl), _p(prefix_len), max_prefix, _p(tree_off),
                                  _p(parent), _p(tokens), _p(cum_logp), _p(workspace),
                                  workspace.numel() * workspace.element_size(), _t(timer), _stream(stream))
    _check(st, "eagle_draft_expand")


def eagle_draft_pool(dims, params, batch, max_prefix, workspace, pool_n=None, token=None, parent=None, depth=None,
                     cum_logp=None, logp=None, expanded=None, *, stream=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    params = draft_params_struct(params)
    st = lib().eagle_draft_pool(ctypes.byref(d), ctypes.byref(params), batch, max_prefix, _p(workspace),
                                workspace.numel() * workspace.element_size(), _p(pool_n), _p(token), _p(parent),
                                _p(depth), _p(cum_logp), _p(logp), _p(expanded), _stream(stream))
    _check(st, "eagle_draft_pool")


def eagle_workspace_size(which, dims, batch, total_nodes, max_nodes, max_prefix, params=None):
    d = dims_struct(dims) if not isinstance(dims, EagleDims) else dims
    params = draft_params_struct(params) if params is not None else None
    return int(lib().eagle_workspace_size(which, ctypes.byref(d), batch, total_nodes, max_nodes, max_prefix,
                                          ctypes.byref(params) if params is not None else None))


def eagle_pack_fragments(w, out=None, stream=None):
    """Fragment-blocked copy of a row-major bf16 matrix w [rows][cols] (eagle_pack_fragments);
    out (allocated when None) holds ceil(rows / 16) * 16 * cols bf16 elements."""
    import torch
    rows, cols = w.shape
    n = (rows + 15) // 16 * 16 * cols
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=w.device)
    if out.numel() < n or w.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or not w.is_contiguous():
        raise EagleError(EAGLE_ERR_ARG, "eagle_pack_fragments")
    _check(lib().eagle_pack_fragments(_p(w), rows, cols, _p(out), _stream(stream)), "eagle_pack_fragments")
    return out


def eagle_fuse_features(dims, w_fuse, feats, root_feature, workspace, *, w_layout=0, stream=None):
    """EAGLE-3 draft input (eagle_fuse_features): root_feature [B][H] f32 = W_fuse [B][3H] feats."""
    d = dims if isinstance(dims, EagleDims) else dims_struct(dims)
    B = feats.shape[0]
    _check(lib().eagle_fuse_features(ctypes.byref(d), _p(w_fuse), int(w_layout), _p(feats), B, _p(root_feature),
                                     _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_fuse_features")


def eagle_workspace_init(workspace, stream=None):
    _check(lib().eagle_workspace_init(_p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_workspace_init")


class Timer:
    """Per-kernel HIP event timing through eagle_timer_*."""

    def __init__(self, capacity=4096, stages=None):
        self.handle = lib().eagle_timer_create(capacity)
        if not self.handle:
            raise RuntimeError("eagle_timer_create failed")
        if stages is not None:
            mask = 0
            for st in stages:
                mask |= 1 << STAGES.index(st)
            _check(lib().eagle_timer_select(self.handle, mask), "eagle_timer_select")

    def collect(self):
        ms = (ctypes.c_double * N_STAGES)()
        cnt = (ctypes.c_int32 * N_STAGES)()
        _check(lib().eagle_timer_collect(self.handle, ms, cnt), "eagle_timer_collect")
        return {STAGES[i]: (ms[i], cnt[i]) for i in range(N_STAGES) if cnt[i]}

    def close(self):
        if self.handle:
            lib().eagle_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
