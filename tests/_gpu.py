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


class HipPathRun:
    """One verification of a workload on the GPU, with debug outputs."""

    def __init__(self, wl, *, use_embed=False, want_logits=True, max_prefix=None, layout=0):
        """layout 1: every weight matrix (LM head and layer) fragment-blocked."""
        import torch
        from tree_attention_verification_06_amd.runner import TreeVerifier, with_packed_weights
        self.wl = wl
        self.t = upload(wl)
        d = wl.dims
        M = wl.n_nodes
        self.M = M
        self.max_nodes = max(len(p) for p in wl.parents)
        self.max_prefix = int(wl.prefix_len.max()) if max_prefix is None else max_prefix
        w = with_packed_weights(self.t["weights"]) if layout else self.t["weights"]
        self.v = TreeVerifier(d, w, self.t["k_cache"], self.t["v_cache"], batch=wl.batch, max_total_nodes=M,
                              max_nodes=self.max_nodes, max_prefix=self.max_prefix, lm_layout=layout,
                              weight_layout=layout)
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


# ---- draft expansion -------------------------------------------------------------------

def gpu_draft_outputs(drafter):
    """Compacted trees and the candidate pool of the drafter's last expansion, as numpy."""
    import torch
    pool = {k: v.cpu().numpy() for k, v in drafter.pool().items()}
    torch.cuda.synchronize()
    tree = dict(tree_off=drafter.tree_off.cpu().numpy(), parent=drafter.parent.cpu().numpy(),
                tokens=drafter.tokens.cpu().numpy(), cum=drafter.cum.cpu().numpy())
    return tree, pool


def draft_force(pool, b, depth):
    """Teacher-forcing record of sequence b: the GPU's expanded nodes and children tokens per level."""
    pn = int(pool["pool_n"][b])
    tok, par = pool["token"][b], pool["parent"][b]
    force = dict(tokens={}, frontier={})
    for lvl in range(1, depth + 1):
        fr = [int(n) for n in pool["expanded"][b, lvl - 1] if n >= 0]
        if lvl == 1:
            assert fr == [0], fr
        else:
            force["frontier"][lvl] = fr
        force["tokens"][lvl] = [[int(tok[i]) for i in range(pn) if par[i] == n] for n in fr]
    return force


def gpu_pool_dicts(pool, b):
    """The GPU pool of sequence b as the oracle's candidate records (gen = pool order)."""
    pn = int(pool["pool_n"][b])
    return [dict(token=int(pool["token"][b, i]), parent=int(pool["parent"][b, i]), depth=int(pool["depth"][b, i]),
                 cum=float(pool["cum"][b, i]), gen=i) for i in range(pn)]


def check_draft_structure(tree, pool, params, B):
    """Decisions the GPU takes in its own precision, replayed exactly from its own values with the
    oracle's definitions: the next frontier of every level and the final rerank.  Plus the
    layout of the compacted outputs.  No oracle numerics needed, so it runs on every sequence."""
    from oracle.draft import draft_rerank, draft_select_level
    M, F, D = params.max_nodes, params.frontier, params.depth
    log_tau = np.log(np.float32(params.conf_threshold)) if params.conf_threshold > 0 else -np.inf
    off = tree["tree_off"]
    assert off[0] == 0
    for b in range(B):
        pn = int(pool["pool_n"][b])
        recs = gpu_pool_dicts(pool, b)
        logp = pool["logp"][b]
        # generation order: children of each level's expanded nodes, in rank order
        nxt = 1
        for lvl in range(1, D + 1):
            fr = [int(n) for n in pool["expanded"][b, lvl - 1] if n >= 0]
            kids = []
            for n in fr:
                k = list(range(nxt, nxt + params.top_k))
                assert all(recs[i]["parent"] == n and recs[i]["depth"] == lvl for i in k), (b, lvl, n)
                kids += k
                nxt += params.top_k
            if lvl < D:
                border = [i for i in kids if abs(float(logp[i]) - float(log_tau)) < 1e-6]
                assert not border, f"child log-prob within 1e-6 of the threshold: {border}"
                ch = [dict(recs[i], p=1.0 if np.float32(logp[i]) >= log_tau else 0.0) for i in kids]
                sel = draft_select_level(ch, F, 0.5)
                want = [kids[i] for i in sel]
                got = [int(n) for n in pool["expanded"][b, lvl] if n >= 0]
                assert got == want, (b, lvl, got, want)
        assert nxt == pn, (b, nxt, pn)
        par, tok, cum, order = draft_rerank(recs, M)
        n = len(par)
        assert off[b + 1] - off[b] == n == min(M, pn)
        o = off[b]
        assert tree["parent"][o:o + n].tolist() == par
        assert tree["tokens"][o:o + n].tolist() == tok
        assert np.array_equal(tree["cum"][o:o + n], np.array(cum, dtype=np.float32))
    end = off[B]
    assert (tree["parent"][end:] == -1).all() and (tree["tokens"][end:] == 0).all()
    assert np.isneginf(tree["cum"][end:]).all()


def check_draft_numerics(wl, params, pool, seqs, *, label=""):
    """Teacher-forced oracle on sequences ``seqs``: the oracle follows the GPU's decisions and
    computes every value itself.  Each child's log-probability (a logit minus the row's
    log-sum-exp) agrees within the bf16 logits tolerance, i.e. relative to the largest |logit|
    of its parent's row; cum is the fp32 recurrence cum(parent) + min(0, log p) of the GPU's
    own values, bit for bit; each expanded node's children are the oracle's own top-k
    wherever its ranking is decisive.  A rank gap is decisive when it exceeds twice the
    logit error the tolerance allows on that row (2 * TOL_BF16 * max|logit|): no pair of
    values that far apart can swap under the tolerance."""
    from oracle.draft import draft_expand
    sel = np.asarray(seqs)
    force = [draft_force(pool, int(b), params.depth) for b in sel]
    res = draft_expand(wl.dims, params, wl.weights, wl.draft_weights, wl.root_feature[sel], wl.root_token[sel],
                       wl.dk_cache[sel], wl.dv_cache[sel], wl.prefix_len[sel], trace=True, force=force)
    errs = {}
    n_decisive = n_ranks = 0
    for j, b in enumerate(sel):
        r = res[j]
        pn = int(pool["pool_n"][b])
        opool = r["pool"]
        assert len(opool) == pn
        assert [c["token"] for c in opool] == pool["token"][b, :pn].tolist()
        assert [c["parent"] for c in opool] == pool["parent"][b, :pn].tolist()
        glogp, gcum, gpar = pool["logp"][b], pool["cum"][b], pool["parent"][b]
        # cum: exact fp32 recurrence over the GPU's own log-probabilities
        want = np.float32(gcum[gpar[1:pn]]) + np.minimum(np.float32(0), glogp[1:pn])
        want = np.where(want == 0, np.float32(0), want)
        assert np.array_equal(gcum[1:pn], want), label
        scale = np.zeros(pn)
        for lv in r["levels"]:
            for row, n in enumerate(lv["frontier"]):
                for c in lv["children"]:
                    if opool[c]["parent"] == n:
                        scale[c] = lv["zscale"][row]
        ologp = np.array([c.get("logp", 0.0) for c in opool])
        e = np.abs(glogp[1:pn].astype(np.float64) - ologp[1:]) / scale[1:]
        errs[f"logp[{b}]"] = float(e.max())
        errs[f"cum[{b}]"] = rel_err(gcum[:pn], np.array([c["cum"] for c in opool]))
        for lvl, lv in enumerate(r["levels"], start=1):
            for row, (own, vals) in enumerate(lv["own_tops"]):
                got = force[j]["tokens"][lvl][row]
                margin = 2 * TOL_BF16 * lv["zscale"][row]
                for c in range(params.top_k):
                    n_ranks += 1
                    if vals[c] - vals[c + 1] > margin:
                        n_decisive += 1
                        assert set(got[:c + 1]) == set(own[:c + 1].tolist()), (label, b, lvl, row, c, got, own)
    print(label, "draft errors", {k: f"{v:.2e}" for k, v in errs.items()},
          f"decisive ranks {n_decisive}/{n_ranks}", flush=True)
    bad = {k: v for k, v in errs.items() if k.startswith("logp") and not v <= TOL_BF16}
    assert not bad, f"{label} tolerance {TOL_BF16} exceeded: {bad}"
    return errs, n_decisive / max(n_ranks, 1)
