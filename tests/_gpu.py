"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs, and compare."""
import numpy as np

import oracle
from workloads.device import upload

TOL_BF16 = 2e-2   # max |gpu - ref| / max |ref| per tensor, bf16 path
TOL_F32 = 1e-4    # fp32 path
GAP_BF16 = 0.05   # argmax ids are compared where the oracle's top-2 logit gap exceeds this
GAP_F32 = 1e-3    # fp32 path: logit errors are ~1e-6, so far smaller gaps are still decisive


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    return float(np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-30))


def np_of(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def tol(dims):
    return TOL_BF16 if dims.dtype == "bf16" else TOL_F32


class GpuRun:
    """One verification of a workload on the GPU, with debug outputs."""

    def __init__(self, wl, *, use_embed=False, want_logits=True, max_prefix=None):
        import torch
        from tree_attention_verification_06_amd.runner import TreeVerifier
        self.wl = wl
        self.t = upload(wl)
        d = wl.dims
        M = wl.n_nodes
        self.M = M
        self.max_nodes = max(len(p) for p in wl.parents)
        self.max_prefix = int(wl.prefix_len.max()) if max_prefix is None else max_prefix
        self.v = TreeVerifier(d, self.t["weights"], self.t["k_cache"], self.t["v_cache"], batch=wl.batch,
                              max_total_nodes=M, max_nodes=self.max_nodes, max_prefix=self.max_prefix)
        self.dbg_attn = torch.zeros(M, d.n_q_heads * d.head_dim, dtype=torch.float32, device="cuda")
        self.dbg_logits = torch.zeros(M, d.vocab, dtype=torch.float32, device="cuda") if want_logits else None
        self.use_embed = use_embed

    def run(self, accept=False):
        import torch
        t, v = self.t, self.v
        v.encode(t["tree_off"], t["parent"], t["prefix_len"], self.M)
        v.verify(t["tree_off"], t["tokens"], t["prefix_len"], self.M,
                 x=None if self.use_embed else t["x"], dbg_attn=self.dbg_attn, dbg_logits=self.dbg_logits)
        if accept:
            v.accept(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"])
        torch.cuda.synchronize()
        return self

    def outputs(self):
        v = self.v
        out = dict(anc=v.anc.cpu().numpy().view(np.uint64), depth=v.depth.cpu().numpy(), pos=v.pos.cpu().numpy(),
                   k_tree=np_of(v.k_tree), v_tree=np_of(v.v_tree), h=np_of(v.h), argmax=np_of(v.argmax),
                   maxlogit=np_of(v.maxlogit), attn=np_of(self.dbg_attn), status=int(v.status.item()))
        if self.dbg_logits is not None:
            out["logits"] = np_of(self.dbg_logits)
        return out


def oracle_verify(wl, use_embed=False, want_logits=True):
    return oracle.verify_forward(wl.dims, wl.weights, None if use_embed else wl.x, wl.parents, wl.prefix_len,
                                 wl.k_cache, wl.v_cache, embed_tokens=wl.tokens if use_embed else None,
                                 want_logits=want_logits)


def check_verify(g, ref, dims, *, label=""):
    """Compare GPU outputs with the oracle: tolerances per tensor, exact argmax where decisive."""
    tl = tol(dims)
    errs = {}
    errs["k_tree"] = rel_err(g["k_tree"], ref["k_tree"])
    errs["v_tree"] = rel_err(g["v_tree"], ref["v_tree"])
    errs["attn"] = rel_err(g["attn"], ref["attn"])
    errs["h"] = rel_err(g["h"], ref["h"])
    errs["maxlogit"] = rel_err(g["maxlogit"], ref["maxlogit"])
    if "logits" in g and "logits" in ref:
        errs["logits"] = rel_err(g["logits"], ref["logits"])
    print(label, "max rel err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tl}
    assert not bad, f"{label} tolerance {tl} exceeded: {bad} (all: {errs})"
    decisive = ref["gap"] > (GAP_BF16 if dims.dtype == "bf16" else GAP_F32)
    mism = np.nonzero(decisive & (g["argmax"] != ref["argmax"]))[0]
    assert len(mism) == 0, f"{label} argmax mismatch at rows {mism[:10]} (gap {ref['gap'][mism[:10]]})"
    assert decisive.mean() > 0.5, f"{label}: too few decisive rows ({decisive.mean():.2f})"
    return errs
