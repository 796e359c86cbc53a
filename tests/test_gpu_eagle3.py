"""GPU parity of the EAGLE-3 draft input (eagle_fuse_features) and of a draft expansion
started from fused root features.

The fusion's inputs are bf16 and their products exact in fp32, so the only error is the
fp32 accumulation over K = 3H terms: typically ~sqrt(K) * 2^-24 of the output scale
(~1e-6 at K = 12288); the tolerance is 1e-4 of max |reference|."""
import numpy as np
import pytest

import oracle
from tests._gpu import check_draft_numerics, check_draft_structure, gpu_draft_outputs
from workloads import DraftParams, make_workload
from workloads.configs import eagle3_inputs, mini_dims
from workloads.device import upload

pytestmark = pytest.mark.gpu
TOL_FUSE = 1e-4


def _log(*a):
    print(*a, flush=True)


def _fuse(wl, w_fuse, feats, layout):
    import torch
    import tree_attention_verification_06_amd as E
    H, B = wl.dims.hidden, wl.batch
    w = torch.from_numpy(w_fuse.view(np.int16)).cuda().view(torch.bfloat16)
    x = torch.from_numpy(feats.view(np.int16)).cuda().view(torch.bfloat16)
    if layout:
        w = E.eagle_pack_fragments(w)
    out = torch.zeros(B, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(E.eagle_workspace_size(2, wl.dims, B, 0, 0, 0), dtype=torch.uint8, device="cuda")
    E.eagle_workspace_init(ws)
    E.eagle_fuse_features(wl.dims, w, x, out, ws, w_layout=layout)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(wl, w_fuse, feats):
    H = wl.dims.hidden
    return oracle.fuse_features(w_fuse, feats[:, :H], feats[:, H:2 * H], feats[:, 2 * H:])


@pytest.mark.parametrize("full", [False, True])
def test_fuse_features_matches_oracle(full):
    if full:
        wl = make_workload(5)  # 8B shape, batch 16: K = 12288
    else:
        wl = make_workload(5, seed=12, dims=mini_dims(), batch=3, prefix=[10, 20, 30],
                           draft=DraftParams(depth=2, top_k=2, frontier=2, max_nodes=4))
    w_fuse, feats = eagle3_inputs(wl)
    ref = _ref(wl, w_fuse, feats)
    got = _fuse(wl, w_fuse, feats, 0)
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    _log(f"fuse {wl.dims.hidden}x{3 * wl.dims.hidden}, batch {wl.batch}: max rel err {err:.2e}")
    assert err <= TOL_FUSE
    packed = _fuse(wl, w_fuse, feats, 1)
    assert np.array_equal(got, packed)  # the packed layout gives the same bits


def test_eagle3_draft_from_fused_roots():
    """Fuse on the GPU, draft on the GPU from the fused roots; teacher-forced oracle check of the
    draft (the oracle drafts from the same fused root features) and exact replay of its choices."""
    from tree_attention_verification_06_amd.runner import TreeDrafter
    params = DraftParams(depth=4, top_k=4, frontier=3, max_nodes=16)
    wl = make_workload(5, seed=14, dims=mini_dims(), batch=3, prefix=[37, 100, 0], draft=params)
    w_fuse, feats = eagle3_inputs(wl)
    root = _fuse(wl, w_fuse, feats, 0)
    ref = _ref(wl, w_fuse, feats)
    assert float(np.abs(root - ref).max() / np.abs(ref).max()) <= TOL_FUSE
    wl.root_feature = root.astype(np.float32)
    t = upload(wl)
    d = TreeDrafter(wl.dims, wl.draft, t["weights"], t["draft_weights"], t["dk_cache"], t["dv_cache"],
                    batch=wl.batch, max_prefix=int(wl.prefix_len.max()))
    d.expand(t["root_feature"], t["root_token"], t["prefix_len"])
    tree, pool = gpu_draft_outputs(d)
    check_draft_structure(tree, pool, params, wl.batch)
    check_draft_numerics(wl, params, pool, range(wl.batch), label="eagle3 mini")
