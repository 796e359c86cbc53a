"""The C ABI library loads, exports every function include/eagle.h declares, and rejects bad
arguments on the host with the documented status (no GPU needed: nothing is enqueued)."""
import ctypes
import os
import re

import pytest

import tree_attention_verification_06_amd as E
from tree_attention_verification_06_amd import _abi as A
from workloads.configs import LLAMA8B, TINY

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "eagle.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(A.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    # and the binding covers exactly those names
    assert set(A.PROTOTYPES) == set(names)


def test_version_and_status_strings():
    assert E.lib().eagle_abi_version() == 7
    assert E.status_str(0) == "ok"
    assert "workspace" in E.status_str(A.EAGLE_ERR_WORKSPACE)


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every case below fails argument checks first


def _tree_build(**kw):
    a = dict(batch=1, tree_off=FAKE, total=5, maxn=5, parent=FAKE, prefix=FAKE, mw=1, anc=FAKE, depth=FAKE,
             pos=FAKE)
    a.update(kw)
    return E.lib().eagle_tree_build(a["batch"], a["tree_off"], a["total"], a["maxn"], a["parent"], a["prefix"],
                                    a["mw"], a["anc"], a["depth"], a["pos"], None, None)


def test_tree_build_host_errors():
    assert _tree_build(batch=0) == A.EAGLE_ERR_ARG
    assert _tree_build(parent=None) == A.EAGLE_ERR_ARG
    assert _tree_build(mw=3) == A.EAGLE_ERR_UNSUPPORTED
    assert _tree_build(maxn=65, mw=1) == A.EAGLE_ERR_CAPACITY


def _verify(dims, ws_bytes=1 << 40, lm_layout=0, layer_layout=0, **kw):
    d = A.dims_struct(dims, lm_layout)
    lw = A.EagleLayerW(4096, 4096, 4096, 4096, 4096, 4096, 4096, layer_layout)
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    a = dict(B=1, total=60, maxn=60, mw=1, max_prefix=2048, ws=ctypes.c_void_p(1 << 20))
    a.update(kw)
    return E.lib().eagle_tree_verify(ctypes.byref(d), ctypes.byref(lw), FAKE, FAKE, a["B"], FAKE, a["total"],
                                     a["maxn"], FAKE, None, None, FAKE, a["mw"], FAKE, FAKE, a["max_prefix"], FAKE,
                                     FAKE, ctypes.byref(cl), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, a["ws"],
                                     ws_bytes, None, None)


def test_verify_host_errors():
    from dataclasses import replace
    assert _verify(LLAMA8B, ws_bytes=16) == A.EAGLE_ERR_WORKSPACE
    assert _verify(replace(LLAMA8B, head_dim=96)) == A.EAGLE_ERR_UNSUPPORTED
    assert _verify(replace(LLAMA8B, n_kv_heads=7)) == A.EAGLE_ERR_UNSUPPORTED
    assert _verify(replace(LLAMA8B, hidden=4000)) == A.EAGLE_ERR_UNSUPPORTED
    assert _verify(LLAMA8B, maxn=65, mw=1) == A.EAGLE_ERR_ARG
    assert _verify(LLAMA8B, B=0) == A.EAGLE_ERR_ARG
    assert _verify(LLAMA8B, ws=ctypes.c_void_p((1 << 20) + 16)) == A.EAGLE_ERR_ARG  # misaligned workspace
    assert _verify(replace(TINY, head_dim=32)) == A.EAGLE_ERR_UNSUPPORTED
    assert _verify(LLAMA8B, lm_layout=2) == A.EAGLE_ERR_ARG
    assert _verify(TINY, lm_layout=1) == A.EAGLE_ERR_UNSUPPORTED  # fragment blocks are bf16 only
    assert _verify(LLAMA8B, layer_layout=2) == A.EAGLE_ERR_ARG
    assert _verify(TINY, layer_layout=1) == A.EAGLE_ERR_UNSUPPORTED


def test_pack_fragments_host_errors():
    pack = E.lib().eagle_pack_fragments
    assert pack(None, 16, 32, FAKE, None) == A.EAGLE_ERR_ARG
    assert pack(FAKE, 16, 32, None, None) == A.EAGLE_ERR_ARG
    assert pack(FAKE, 0, 32, FAKE, None) == A.EAGLE_ERR_ARG
    assert pack(FAKE, 16, 48, FAKE, None) == A.EAGLE_ERR_ARG    # columns not a multiple of 32
    assert pack(FAKE, 16, 0, FAKE, None) == A.EAGLE_ERR_ARG
    assert pack(ctypes.c_void_p(4096 + 8), 16, 32, FAKE, None) == A.EAGLE_ERR_ARG  # misaligned


def test_workspace_size_query():
    assert E.eagle_workspace_size(0, LLAMA8B, 1, 60, 60, 2048) > 0
    from dataclasses import replace
    assert E.eagle_workspace_size(0, replace(LLAMA8B, head_dim=96), 1, 60, 60, 2048) == 0
    assert E.eagle_workspace_size(7, LLAMA8B, 1, 60, 60, 2048) == 0


def test_accept_host_errors():
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    f = E.lib().eagle_accept_commit

    def call(**kw):
        a = dict(B=1, maxn=60, mw=1, hkv=8, hd=128, dtype=0, max_accept=16, tree_off=FAKE)
        a.update(kw)
        return f(a["B"], a["tree_off"], a["maxn"], FAKE, FAKE, FAKE, FAKE, a["mw"], FAKE, FAKE, FAKE, FAKE, FAKE,
                 ctypes.byref(cl), a["hkv"], a["hd"], a["dtype"], FAKE, None, 4096, None, a["max_accept"], FAKE,
                 FAKE, FAKE, FAKE, None, None)
    assert call(B=0) == A.EAGLE_ERR_ARG
    assert call(tree_off=None) == A.EAGLE_ERR_ARG
    assert call(maxn=130, mw=2) == A.EAGLE_ERR_CAPACITY
    assert call(dtype=5) == A.EAGLE_ERR_UNSUPPORTED
    assert call(max_accept=500) == A.EAGLE_ERR_ARG
    assert call(hd=4) == A.EAGLE_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        A.lib()


def test_fuse_features_host_errors():
    from dataclasses import replace
    L = E.lib()
    ws_bytes = A.eagle_workspace_size(2, LLAMA8B, 16, 0, 0, 0)
    assert ws_bytes > 0
    assert A.eagle_workspace_size(2, TINY, 16, 0, 0, 0) == 0  # fp32 dims: unsupported
    d = A.dims_struct(LLAMA8B)
    ws = ctypes.c_void_p(1 << 20)

    def fuse(dims=d, w=FAKE, layout=0, x=FAKE, b=16, out=FAKE, w_s=ws, nbytes=ws_bytes):
        return L.eagle_fuse_features(ctypes.byref(dims), w, layout, x, b, out, w_s, nbytes, None)
    assert fuse(w=None) == A.EAGLE_ERR_ARG
    assert fuse(out=None) == A.EAGLE_ERR_ARG
    assert fuse(b=0) == A.EAGLE_ERR_ARG
    assert fuse(layout=2) == A.EAGLE_ERR_ARG
    assert fuse(w_s=ctypes.c_void_p((1 << 20) + 16)) == A.EAGLE_ERR_ARG  # misaligned workspace
    assert fuse(nbytes=ws_bytes - 1) == A.EAGLE_ERR_WORKSPACE
    assert fuse(dims=A.dims_struct(TINY)) == A.EAGLE_ERR_UNSUPPORTED
    assert fuse(dims=A.dims_struct(replace(LLAMA8B, hidden=4000))) == A.EAGLE_ERR_UNSUPPORTED



def test_verify_sample_host_errors():
    from dataclasses import replace
    L = E.lib()
    d = A.dims_struct(LLAMA8B)
    lw = A.EagleLayerW(4096, 4096, 4096, 4096, 4096, 4096, 4096, 0)
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    ws_bytes = A.eagle_workspace_size(3, LLAMA8B, 1, 60, 60, 2048)
    assert ws_bytes > A.eagle_workspace_size(0, LLAMA8B, 1, 60, 60, 2048) > 0
    ws = ctypes.c_void_p(1 << 20)

    def call(dims=d, temperature=1.0, gumbel=FAKE, tokens=FAKE, parent=FAKE, out=FAKE, nbytes=ws_bytes):
        return L.eagle_tree_verify_sample(ctypes.byref(dims), ctypes.byref(lw), FAKE, FAKE, 1, FAKE, 60, 60, FAKE,
                                          None, tokens, parent, FAKE, 1, FAKE, FAKE, 2048, FAKE, FAKE,
                                          ctypes.byref(cl), temperature, gumbel, FAKE, FAKE, FAKE, out, FAKE, FAKE,
                                          ws, nbytes, None, None)
    assert call(temperature=0.0) == A.EAGLE_ERR_ARG
    assert call(temperature=-1.0) == A.EAGLE_ERR_ARG
    assert call(temperature=float("nan")) == A.EAGLE_ERR_ARG
    assert call(temperature=1e-45) == A.EAGLE_ERR_ARG  # 1/T overflows
    assert call(gumbel=None) == A.EAGLE_ERR_ARG
    assert call(tokens=None) == A.EAGLE_ERR_ARG
    assert call(parent=None) == A.EAGLE_ERR_ARG
    assert call(out=None) == A.EAGLE_ERR_ARG
    assert call(nbytes=ws_bytes - 1) == A.EAGLE_ERR_WORKSPACE
    assert call(dims=A.dims_struct(replace(LLAMA8B, head_dim=96))) == A.EAGLE_ERR_UNSUPPORTED


def test_accept_sample_host_errors():
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    f = E.lib().eagle_accept_commit_sample

    def call(**kw):
        a = dict(B=1, maxn=60, hkv=8, hd=128, dtype=0, max_accept=16, tree_off=FAKE, u=FAKE, cl=FAKE)
        a.update(kw)
        return f(a["B"], a["tree_off"], a["maxn"], FAKE, FAKE, a["cl"], FAKE, FAKE, a["u"], FAKE, FAKE, FAKE, FAKE,
                 ctypes.byref(cl), a["hkv"], a["hd"], a["dtype"], FAKE, None, 4096, None, a["max_accept"], FAKE,
                 FAKE, FAKE, FAKE, None, None)
    assert call(B=0) == A.EAGLE_ERR_ARG
    assert call(tree_off=None) == A.EAGLE_ERR_ARG
    assert call(u=None) == A.EAGLE_ERR_ARG
    assert call(cl=None) == A.EAGLE_ERR_ARG
    assert call(maxn=129) == A.EAGLE_ERR_CAPACITY
    assert call(dtype=5) == A.EAGLE_ERR_UNSUPPORTED
    assert call(max_accept=500) == A.EAGLE_ERR_ARG
    assert call(hd=4) == A.EAGLE_ERR_UNSUPPORTED


def test_verify_layers_host_errors():
    from dataclasses import replace
    L = E.lib()
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    ws_bytes = A.eagle_workspace_size(0, LLAMA8B, 1, 60, 60, 2048)
    ws = ctypes.c_void_p(1 << 20)

    def call(dims=LLAMA8B, n=2, arr_n=2, stride=1 << 24, gates=True, nbytes=ws_bytes):
        d = A.dims_struct(dims)
        lws = [A.EagleLayerW(4096, 4096, 4096, 4096, 4096 if gates else None, 4096, 4096, 0) for _ in range(arr_n)]
        arr = (A.EagleLayerW * arr_n)(*lws)
        return L.eagle_tree_verify_layers(ctypes.byref(d), n, arr, FAKE, FAKE, 1, FAKE, 60, 60, FAKE, None, None,
                                          FAKE, 1, FAKE, FAKE, 2048, FAKE, FAKE, ctypes.byref(cl), stride, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, None, None, ws, nbytes, None, None)
    assert call(n=0) == A.EAGLE_ERR_ARG
    assert call(n=2000, arr_n=2) == A.EAGLE_ERR_ARG
    assert call(stride=-1) == A.EAGLE_ERR_ARG
    assert call(gates=False) == A.EAGLE_ERR_ARG  # a layer without its MLP matrices
    assert call(dims=TINY) == A.EAGLE_ERR_UNSUPPORTED  # a stack needs the MLP layer
    assert call(dims=replace(LLAMA8B, head_dim=96)) == A.EAGLE_ERR_UNSUPPORTED
    assert call(nbytes=ws_bytes - 1) == A.EAGLE_ERR_WORKSPACE


def test_accept_commit_layers_host_errors():
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    f = E.lib().eagle_accept_commit_layers

    def call(**kw):
        a = dict(B=1, maxn=60, mw=1, n=4, cs=1 << 24, ts=1 << 20, dtype=0, tree_off=FAKE)
        a.update(kw)
        return f(a["B"], a["tree_off"], a["maxn"], FAKE, FAKE, FAKE, FAKE, a["mw"], FAKE, FAKE, FAKE, FAKE, FAKE,
                 ctypes.byref(cl), 8, 128, a["dtype"], a["n"], a["cs"], a["ts"], FAKE, None, 4096, None, 16, FAKE,
                 FAKE, FAKE, FAKE, None, None)
    assert call(n=0) == A.EAGLE_ERR_ARG
    assert call(cs=0) == A.EAGLE_ERR_ARG
    assert call(ts=-64) == A.EAGLE_ERR_ARG
    assert call(ts=3) == A.EAGLE_ERR_ARG  # not a multiple of 16 bytes
    assert call(tree_off=None) == A.EAGLE_ERR_ARG
    assert call(maxn=130, mw=2) == A.EAGLE_ERR_CAPACITY
    assert call(dtype=5) == A.EAGLE_ERR_UNSUPPORTED


def test_draft_kv_commit_host_errors():
    from dataclasses import replace
    L = E.lib()
    cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
    ws_bytes = A.eagle_workspace_size(4, LLAMA8B, 16, 0, 7, 0)
    assert ws_bytes > 0
    assert A.eagle_workspace_size(4, TINY, 16, 0, 7, 0) == 0
    ws = ctypes.c_void_p(1 << 20)
    lw = A.EagleLayerW(4096, 4096, 4096, 4096, 4096, 4096, 4096, 0)

    def call(dims=LLAMA8B, w_fc=FAKE, h=FAKE, root=FAKE, max_accept=6, w_s=ws, nbytes=ws_bytes):
        d = A.dims_struct(dims)
        return L.eagle_draft_kv_commit(ctypes.byref(d), w_fc, ctypes.byref(lw), FAKE, 16, FAKE, FAKE, h, root, FAKE,
                                       FAKE, max_accept, FAKE, FAKE, FAKE, ctypes.byref(cl), None, w_s, nbytes, None)
    assert call(w_fc=None) == A.EAGLE_ERR_ARG
    assert call(h=None) == A.EAGLE_ERR_ARG
    assert call(root=None) == A.EAGLE_ERR_ARG
    assert call(max_accept=-1) == A.EAGLE_ERR_ARG
    assert call(max_accept=128) == A.EAGLE_ERR_ARG
    assert call(w_s=ctypes.c_void_p((1 << 20) + 16)) == A.EAGLE_ERR_ARG
    assert call(nbytes=ws_bytes - 1) == A.EAGLE_ERR_WORKSPACE
    assert call(dims=TINY) == A.EAGLE_ERR_UNSUPPORTED
    assert call(dims=replace(LLAMA8B, head_dim=64)) == A.EAGLE_ERR_UNSUPPORTED


def test_paged_cache_layout_host_errors():
    """A block table needs a page size that is a positive multiple of 64, positive
    max_blocks and n_pages, and capacity <= max_blocks * page_size."""
    cases = [(dict(), A.EAGLE_OK), (dict(page_size=48), A.EAGLE_ERR_ARG), (dict(page_size=0), A.EAGLE_ERR_ARG),
             (dict(max_blocks=0), A.EAGLE_ERR_ARG), (dict(n_pages=0), A.EAGLE_ERR_ARG),
             (dict(capacity=64 * 33), A.EAGLE_ERR_ARG)]
    L = E.lib()
    d = A.dims_struct(LLAMA8B)
    lw = A.EagleLayerW(4096, 4096, 4096, 4096, 4096, 4096, 4096, 0)
    for kw, want in cases:
        f = dict(capacity=64 * 32, page_size=64, max_blocks=32, n_pages=100)
        f.update(kw)
        cl = A.EagleCacheLayout(1 << 20, 1 << 13, 128, f["capacity"], 4096, f["page_size"], f["max_blocks"],
                                f["n_pages"])
        # a workspace that is too small: a valid layout gets as far as the workspace check
        st = L.eagle_tree_verify(ctypes.byref(d), ctypes.byref(lw), FAKE, FAKE, 1, FAKE, 60, 60, FAKE, None, None, FAKE,
                                 1, FAKE, FAKE, 2048, FAKE, FAKE, ctypes.byref(cl), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 None, ctypes.c_void_p(1 << 20), 16, None, None)
        assert st == (A.EAGLE_ERR_WORKSPACE if want == A.EAGLE_OK else want), (kw, st)
        st = L.eagle_accept_commit(1, FAKE, 60, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(cl),
                                   8, 128, 0, FAKE, None, 4096, None, 16, FAKE, FAKE, FAKE, FAKE, None, None)
        if want != A.EAGLE_OK:
            assert st == want, (kw, st)


def test_verify_noalloc_refuses_oversized_requests_on_the_host():
    """The entry point that allocates nothing refuses, before touching the GPU, any shape
    whose scratch would exceed the library's per-GPU buffer (here the 8B layer with 16 trees
    of 60 nodes: 162 MiB against 32 MiB), and runs the ordinary argument checks first."""
    from workloads.configs import LLAMA8B
    need = A.eagle_workspace_size(0, LLAMA8B, 16, 960, 60, 2048)
    assert need > A.NOALLOC_MAX_BYTES
    assert A.eagle_workspace_size(0, LLAMA8B, 1, 60, 60, 2048) <= A.NOALLOC_MAX_BYTES

    def call(B, total, maxn, w_lm=FAKE):
        d = A.dims_struct(LLAMA8B)
        lw = A.EagleLayerW(4096, 4096, 4096, 4096, 4096, 4096, 4096, 0)
        cl = A.EagleCacheLayout(1 << 20, 1 << 16, 128, 4096)
        return E.lib().eagle_tree_verify_noalloc(ctypes.byref(d), ctypes.byref(lw), FAKE, w_lm, B, FAKE, total, maxn,
                                                 FAKE, None, None, FAKE, 1, FAKE, FAKE, 2048, FAKE, FAKE,
                                                 ctypes.byref(cl), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None)
    assert call(16, 960, 60) == A.EAGLE_ERR_WORKSPACE
    assert call(1, 60, 60, w_lm=None) == A.EAGLE_ERR_ARG
    assert call(0, 60, 60) == A.EAGLE_ERR_ARG
