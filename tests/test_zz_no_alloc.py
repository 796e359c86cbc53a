"""The verification entry point that allocates nothing (eagle_tree_verify_noalloc) against
eagle_tree_verify with a caller workspace: same kernels, so the outputs must agree bit for
bit, on two calls in a row, the second with a smaller batch, fewer nodes and a shorter
prefix (the library's scratch keeps the first call's contents), and the GPU outputs are
also within the bf16 tolerance of the oracle."""
import numpy as np
import pytest

from tests._gpu import HipPathRun, check_verify, oracle_verify
from workloads import make_workload, mini_dims, trees as T

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    t = t.contiguous().cpu()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).numpy()


def _noalloc_outputs(run):
    """The same verification as run.run(), through the entry point without a workspace."""
    import torch
    import tree_attention_verification_06_amd as E
    v, t, d = run.v, run.t, run.wl.dims
    M = run.M
    z = lambda *s, dtype: torch.zeros(*s, dtype=dtype, device="cuda")  # noqa: E731
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    out = dict(k_tree=z(M, d.n_kv_heads, d.head_dim, dtype=dt), v_tree=z(M, d.n_kv_heads, d.head_dim, dtype=dt),
               h=z(M, d.hidden, dtype=torch.float32), argmax=z(M, dtype=torch.int32),
               maxlogit=z(M, dtype=torch.float32), attn=z(M, d.n_q_heads * d.head_dim, dtype=torch.float32),
               logits=z(M, d.vocab, dtype=torch.float32))
    E.eagle_tree_verify_noalloc(v.dstruct, v.lstruct, v.w.get("final_ln"), v.w["w_lm"], t["tree_off"], t["x"], None,
                                t["tokens"], v.anc, v.mw, v.pos, t["prefix_len"], v.k_cache, v.v_cache, out["k_tree"],
                                out["v_tree"], out["h"], out["argmax"], out["maxlogit"], total_nodes=M,
                                max_nodes=run.max_nodes, max_prefix=run.max_prefix, dbg_attn=out["attn"],
                                dbg_logits=out["logits"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_verify_equals_workspace_verify_on_two_calls(layout):
    dims = mini_dims()
    big = make_workload(2, seed=41, dims=dims, batch=3, prefix=[700, 129, 2000],
                        parents=[T.static_tree_60(), T.random_tree(np.random.default_rng(2), 45), T.chain(20)])
    small = make_workload(2, seed=43, dims=dims, batch=1, prefix=[90], parents=[T.random_tree(
        np.random.default_rng(5), 17)])
    for wl in (big, small):
        print("noalloc verify", layout, wl.tree_off.tolist(), wl.prefix_len.tolist(), flush=True)
        run = HipPathRun(wl, layout=layout).run()
        ref_gpu = run.outputs()
        got = _noalloc_outputs(run)
        for k in ("k_tree", "v_tree"):
            assert (_bits(got[k]) == _bits(getattr(run.v, k))).all(), k
        for k, gk in (("h", "h"), ("argmax", "argmax"), ("maxlogit", "maxlogit"), ("attn", "attn"),
                      ("logits", "logits")):
            assert np.array_equal(got[k].cpu().numpy(), ref_gpu[gk]), k
        g = dict(ref_gpu)
        g.update({k: (got[k].float() if k in ("k_tree", "v_tree") else got[k]).cpu().numpy() for k in got})
        check_verify(g, oracle_verify(wl), dims, label=f"noalloc-{layout}")
