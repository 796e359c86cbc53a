"""GPU parity of verification and acceptance at temperature T > 0 (eagle_tree_verify_sample,
eagle_accept_commit_sample) against the fp64 oracle (oracle.sample_summaries,
oracle.sample_accept_from_summaries, oracle.sample_accept_sequence).

Node inputs are given hidden states, so the target's logits do not depend on the tree's
tokens: the oracle's logits are computed first and each node's children then get the top-k
tokens of their parent's row in random order (a perfect drafter's candidates), so walks go
deep at low temperature.  Checks:
  * per-node summaries against the oracle: child_logit and rest_lse within the logits
    tolerance times the largest |logit / T|; rest_token never a child token, and equal to
    the oracle's wherever its best noisy score beats the runner-up by more than twice the
    GPU's measured logit error dz (the greedy path's debug logits, the same LM-head
    arithmetic, give dz), else one of the near-tied tokens;
  * the same summaries of the GPU's own logits (oracle.sample_summaries on them): within
    1e-5 relative, and rest_token exact unless fp32 rounding could swap the top two;
  * the walk: acceptance uniforms are first moved away from every decision threshold of the
    oracle's walk on the exact logits by a margin the GPU's probability error (from dz)
    cannot cross; the GPU's path, tokens and bonus then equal the oracle's, and the whole
    result equals the oracle's walk replayed on the GPU's own summaries;
  * the commit, bit for bit: cache slots prefix .. prefix + L hold the path's K/V rows, the
    rest of the cache is untouched, prefix_len grows by L + 1, next_feature = h[leaf].
"""
import numpy as np
import pytest

import oracle
from tests._gpu import TOL_BF16, TOL_F32, np_of, oracle_verify
from workloads import make_workload, mini_dims, trees as T
from workloads.configs import sample_inputs

pytestmark = pytest.mark.gpu

EAGLE_ERR_TREE = -2


def _log(*a):
    print(*a, flush=True)


def _plant(wl, logits, rng, trees=None):
    """Children of every node (of trees ``trees``, default all) get the top-k tokens of their
    parent's logits, shuffled."""
    tokens = wl.tokens.copy()
    for b, par in enumerate(wl.parents):
        if trees is not None and b not in trees:
            continue
        o = int(wl.tree_off[b])
        kids = {}
        for j in range(1, len(par)):
            kids.setdefault(par[j], []).append(j)
        for p, ch in kids.items():
            top = np.argsort(-logits[o + p], kind="stable")[:len(ch)]
            rng.shuffle(top)
            for j, tk in zip(ch, top):
                tokens[o + j] = int(tk)
    return tokens


def _nudge(parent, tokens, logits, temperature, u, g, margin):
    """Move u[c] of every decision of the oracle's walk whose |u r - p| < margin * p out of
    that band (keeping its side where possible), until the walk has no such decision."""
    u = np.array(u, dtype=np.float64)
    for _ in range(4 * len(parent) + 4):
        trace = []
        oracle.sample_accept_sequence(parent, tokens, logits, temperature, u, np.broadcast_to(g, logits.shape),
                                      trace=trace)
        near = [(c, ur, p) for c, ur, p in trace if abs(ur - p) < margin * p]
        if not near:
            return u.astype(np.float32)
        c, ur, p = near[0]
        r = ur / u[c] if u[c] > 0 else 1.0
        rej = p * (1.0 + 2.0 * margin) / r
        u[c] = rej if (ur >= p and rej < 1.0) else p * (1.0 - 2.0 * margin) / r
    raise AssertionError("could not move the acceptance uniforms away from the thresholds")


def _one_tree(wl, b):
    """Sequence b of a workload as a workload of its own (trees are independent)."""
    from dataclasses import replace
    o, n = int(wl.tree_off[b]), len(wl.parents[b])
    return replace(wl, batch=1, parents=[wl.parents[b]], tree_off=np.array([0, n], dtype=np.int32),
                   tokens=wl.tokens[o:o + n], x=wl.x[o:o + n], prefix_len=wl.prefix_len[b:b + 1],
                   k_cache=wl.k_cache[b:b + 1], v_cache=wl.v_cache[b:b + 1])


def _run(wl, *, temperature, plant=True, draw=0, pad=0, layout=0, tokens=None, trees=None):
    """trees: the sequences the oracle computes (default all; the GPU always runs the whole
    batch); logits rows of the other sequences are NaN."""
    import torch
    from tree_attention_verification_06_amd.runner import TreeVerifier, with_packed_weights
    from workloads.device import to_tensor, upload
    d = wl.dims
    if trees is None:
        ref = oracle_verify(wl, want_logits=True)
        logits = ref["logits"]
    else:
        ref = None
        logits = np.full((wl.n_nodes, d.vocab), np.nan)
        for b in trees:
            o, n = int(wl.tree_off[b]), len(wl.parents[b])
            logits[o:o + n] = oracle_verify(_one_tree(wl, b), want_logits=True)["logits"]
            _log(f"oracle tree {b} done")
    sel = list(range(wl.batch)) if trees is None else list(trees)
    rows = np.concatenate([np.arange(int(wl.tree_off[b]), int(wl.tree_off[b + 1])) for b in sel])
    rng = np.random.default_rng([wl.seed, 99, draw])
    if tokens is None:
        tokens = _plant(wl, logits, rng, trees) if plant else wl.tokens.copy()
    gumbel, u = sample_inputs(wl, draw)
    tl = TOL_BF16 if d.dtype == "bf16" else TOL_F32

    t = upload(wl)
    n0 = wl.n_nodes
    M = n0 + pad
    parent = np.concatenate([np.asarray(p, dtype=np.int32) for p in wl.parents] + [np.full(pad, -1, np.int32)])
    tok_p = np.concatenate([tokens, np.zeros(pad, np.int32)]).astype(np.int32)
    x = wl.x if pad == 0 else np.concatenate([wl.x, np.zeros((pad, d.hidden), dtype=wl.x.dtype)])
    t_parent, t_tok, t_x = to_tensor(parent, "cuda"), to_tensor(tok_p, "cuda"), to_tensor(x, "cuda")
    t_g = to_tensor(gumbel, "cuda")
    max_nodes = max(len(p) for p in wl.parents)
    w = with_packed_weights(t["weights"]) if layout else t["weights"]
    v = TreeVerifier(d, w, t["k_cache"], t["v_cache"], batch=wl.batch, max_total_nodes=M, max_nodes=max_nodes,
                     max_prefix=int(wl.prefix_len.max()), lm_layout=layout, weight_layout=layout, sample=True)
    v.encode(t["tree_off"], t_parent, t["prefix_len"], M)
    # the GPU's full logits from the greedy path (same LM-head arithmetic): how far its
    # logits are from the oracle's, and a tight reference for the sampling summaries
    dbg = torch.zeros(M, d.vocab, dtype=torch.float32, device="cuda")
    v.verify(t["tree_off"], t_tok, t["prefix_len"], M, x=t_x, dbg_logits=dbg)
    torch.cuda.synchronize()
    gpu_logits = np.full((n0, d.vocab), np.nan)
    gpu_logits[rows] = np_of(dbg[torch.from_numpy(rows).cuda()]).astype(np.float64)
    del dbg
    dz = float(np.abs(gpu_logits[rows] - logits[rows]).max()) / temperature
    # u away from the oracle's thresholds by more than the GPU's probabilities can be off
    margin = min(0.45, 4.0 * (np.exp(2.0 * dz) - 1.0) + 1e-4)
    for b in sel:
        par = wl.parents[b]
        o, n = int(wl.tree_off[b]), len(par)
        u[o:o + n] = _nudge(par, tokens[o:o + n], logits[o:o + n], temperature, u[o:o + n], gumbel[b], margin)
    t_u = to_tensor(np.concatenate([u, np.zeros(pad, np.float32)]), "cuda")

    v.verify_sample(t["tree_off"], t_tok, t_parent, t["prefix_len"], M, temperature, t_g, x=t_x)
    torch.cuda.synchronize()
    summ = dict(child_logit=np_of(v.child_logit), rest_lse=np_of(v.rest_lse), rest_token=np_of(v.rest_token),
                h=np_of(v.h), k_tree=np_of(v.k_tree), v_tree=np_of(v.v_tree))
    kc0, vc0 = np_of(t["k_cache"]).copy(), np_of(t["v_cache"]).copy()
    v.accept_sample(t["tree_off"], t_parent, t_tok, t_u, t["prefix_len"])
    torch.cuda.synchronize()
    acc = dict(accept_len=np_of(v.accept_len), path=np_of(v.path), out_tokens=np_of(v.out_tokens),
               next_token=np_of(v.next_token), next_feature=np_of(v.next_feature), status=int(v.status.item()),
               prefix_len=np_of(t["prefix_len"]), k_cache=np_of(t["k_cache"]), v_cache=np_of(t["v_cache"]))
    return dict(ref=ref, logits=logits, gpu_logits=gpu_logits, dz=dz, tokens=tokens, gumbel=gumbel, u=u,
                err=tl * float(np.abs(logits[rows]).max()) / temperature, summ=summ, acc=acc, kc0=kc0, vc0=vc0,
                trees=sel)


def _check(wl, r, temperature, label):
    """Every check of the module docstring on one run."""
    summ, acc, logits, tokens, err, dz = r["summ"], r["acc"], r["logits"], r["tokens"], r["err"], r["dz"]
    assert acc["status"] == 0, acc["status"]
    worst = {"child_logit": 0.0, "rest_lse": 0.0}
    tight = {"child_logit": 0.0, "rest_lse": 0.0}
    n_dec = n_tok = 0
    depths = []
    V = logits.shape[1]
    for b, par in enumerate(wl.parents):
        o, n = int(wl.tree_off[b]), len(par)
        tk = tokens[o:o + n]
        g = r["gumbel"][b].astype(np.float64)
        g_cl = summ["child_logit"][o:o + n].astype(np.float64)
        g_rl = summ["rest_lse"][o:o + n].astype(np.float64)
        g_rt = summ["rest_token"][o:o + n]
        u = r["u"][o:o + n].astype(np.float64)
        if b not in r["trees"]:
            # no oracle logits for this sequence: the walk and commit against the oracle's
            # walk on the GPU's own summaries
            L, path, out, bonus, leaf = oracle.sample_accept_from_summaries(par, tk, g_cl, g_rl, g_rt, u)
            _check_commit(wl, r, b, L, path, out, bonus, leaf, label)
            continue
        cl, rl, rt = oracle.sample_summaries(par, tk, logits[o:o + n], temperature, g)
        # the same summaries of the GPU's own logits: what the epilogue and merge must give up
        # to fp32 rounding
        tcl, trl, trt = oracle.sample_summaries(par, tk, r["gpu_logits"][o:o + n], temperature, g)
        if n > 1:
            worst["child_logit"] = max(worst["child_logit"], float(np.abs(g_cl[1:] - cl[1:]).max()))
            tight["child_logit"] = max(tight["child_logit"],
                                       float((np.abs(g_cl[1:] - tcl[1:]) / np.maximum(1.0, np.abs(tcl[1:]))).max()))
        worst["rest_lse"] = max(worst["rest_lse"], float(np.abs(g_rl - rl).max()))
        tight["rest_lse"] = max(tight["rest_lse"], float((np.abs(g_rl - trl) / np.maximum(1.0, np.abs(trl))).max()))
        z = logits[o:o + n] / temperature
        zg = r["gpu_logits"][o:o + n] / temperature
        for i in range(n):
            kids = [int(tk[c]) for c in range(1, n) if par[c] == i]
            assert int(g_rt[i]) not in kids, (label, b, i)
            # against the GPU's own logits: exact unless fp32 rounding could swap the top two
            sg = zg[i] + g
            sg[kids] = -np.inf
            top2 = np.sort(sg)[-2:]
            if top2[1] - top2[0] > 1e-5 * max(1.0, abs(top2[1])):
                assert int(g_rt[i]) == int(trt[i]), (label, b, i)
            # against the oracle: exact wherever the GPU's logit error cannot swap the top two
            score = z[i] + g
            score[kids] = -np.inf
            best = score.max()
            second = np.partition(score, -2)[-2] if V > 1 else -np.inf
            n_tok += 1
            if best - second > 2.0 * dz:
                n_dec += 1
                assert int(g_rt[i]) == int(rt[i]), (label, b, i, int(g_rt[i]), int(rt[i]))
            else:
                assert score[int(g_rt[i])] >= best - 2.0 * dz - 1e-9, (label, b, i)
        # the walk: the oracle on the exact logits (u is clear of its thresholds) ...
        L, path, out, bonus, leaf = oracle.sample_accept_sequence(par, tk, logits[o:o + n], temperature, u,
                                                                  np.broadcast_to(g, (n, V)))
        depths.append(int(acc["accept_len"][b]))
        _check_commit(wl, r, b, L, path, out[:L] + [int(g_rt[leaf])], None, leaf, label)
        # ... and the oracle replayed on the GPU's own summaries, decision for decision
        rL, rpath, rout, rbonus, _ = oracle.sample_accept_from_summaries(par, tk, g_cl, g_rl, g_rt, u)
        assert (rL, rpath, rout) == (L, path, acc["out_tokens"][b, :L + 1].tolist()), (label, b)
    _log(label, f"T={temperature}", "max |err| vs oracle", {k: f"{v:.2e}" for k, v in worst.items()},
         f"bound {err:.2e}", "vs own logits", {k: f"{v:.1e}" for k, v in tight.items()}, f"dz {dz:.2e}",
         f"decisive bonus rows {n_dec}/{n_tok}", "accept", depths)
    for k, v in worst.items():
        assert v <= err, (label, k, v, err)
    for k, v in tight.items():
        assert v <= 1e-5, (label, k, v)
    assert n_dec >= 0.5 * n_tok, (label, n_dec, n_tok)
    return depths


def _check_commit(wl, r, b, L, path, out, bonus, leaf, label):
    """Sequence b's outputs are (L, path, out) and its commit is bit-exact: cache slots
    prefix .. prefix + L hold the path's K/V rows, nothing else changed, prefix_len grew by
    L + 1 and next_feature is h[leaf].  bonus None: the bonus is out[L]."""
    acc, summ = r["acc"], r["summ"]
    o = int(wl.tree_off[b])
    gL = int(acc["accept_len"][b])
    assert gL == L, (label, b, gL, L)
    assert acc["path"][b, :L + 1].tolist() == path and (acc["path"][b, L + 1:] == -1).all(), (label, b)
    assert acc["out_tokens"][b, :L + 1].tolist() == out and (acc["out_tokens"][b, L + 1:] == -1).all(), (label, b)
    assert int(acc["next_token"][b]) == (out[L] if bonus is None else bonus), (label, b)
    P = int(wl.prefix_len[b])
    assert acc["prefix_len"][b] == P + L + 1
    for dpos, node in enumerate(path):
        assert np.array_equal(acc["k_cache"][b, :, P + dpos], summ["k_tree"][o + node]), (label, b, dpos)
        assert np.array_equal(acc["v_cache"][b, :, P + dpos], summ["v_tree"][o + node]), (label, b, dpos)
    untouched = np.ones(acc["k_cache"].shape[2], dtype=bool)
    untouched[P:P + L + 1] = False
    assert np.array_equal(acc["k_cache"][b][:, untouched], r["kc0"][b][:, untouched])
    assert np.array_equal(acc["v_cache"][b][:, untouched], r["vc0"][b][:, untouched])
    assert np.array_equal(acc["next_feature"][b], summ["h"][o + leaf])


def _mini(seed=7):
    dims = mini_dims()
    rng = np.random.default_rng(1)
    return make_workload(2, seed=seed, dims=dims, batch=4, prefix=[200, 77, 5, 130],
                         parents=[T.static_tree_60(), T.random_tree(rng, 25), [-1], T.random_tree(rng, 40)])


@pytest.mark.parametrize("temperature", [0.1, 1.0])
def test_sample_mini_bf16(temperature):
    wl = _mini()
    r = _run(wl, temperature=temperature)
    depths = _check(wl, r, temperature, "mini bf16")
    if temperature < 0.5:
        assert max(depths) >= 2, depths  # planted candidates at low T: walks go deep


def test_sample_mini_bf16_unplanted_padded_packed():
    """Uniform random tokens (walks stop early), padding rows past the trees, and
    fragment-blocked weights."""
    wl = _mini(seed=8)
    r = _run(wl, temperature=0.7, plant=False, pad=9, layout=1, draw=1)
    _check(wl, r, 0.7, "mini bf16 unplanted")


def test_sample_tiny_fp32():
    wl = make_workload(1)
    r = _run(wl, temperature=0.5)
    _check(wl, r, 0.5, "tiny fp32")


def test_sample_llama8b_60_nodes():
    """The 8B-shaped layer and 128256-token LM head, the benchmark's layout."""
    wl = make_workload(2)
    r = _run(wl, temperature=0.3, layout=1)
    _check(wl, r, 0.3, "8b")


def test_sample_llama8b_batch16():
    """The benchmark's launch configuration: 16 trees of 60 nodes (960 LM-head rows, the
    wide-tile GEMM) at the 8B shape with fragment-blocked weights.  The GPU runs the whole
    batch; the oracle computes sequences 0 and 9 (trees are independent) and every other
    sequence is checked against the oracle's walk on the GPU's own summaries."""
    wl = make_workload(2, batch=16, parents=[T.static_tree_60() for _ in range(16)])
    r = _run(wl, temperature=0.3, layout=1, trees=[0, 9])
    _check(wl, r, 0.3, "8b batch16")


@pytest.mark.parametrize("trees", [(1, 2, 3, 4, 5), (6, 7, 8, 10, 11), (12, 13, 14, 15)])
def test_sample_llama8b_batch16_other_trees(trees):
    """The same batch; the oracle computes the other fourteen trees, a few per test, so that
    every tree of the 960-row launch is compared with the oracle."""
    wl = make_workload(2, batch=16, parents=[T.static_tree_60() for _ in range(16)])
    r = _run(wl, temperature=0.3, layout=1, trees=list(trees))
    _check(wl, r, 0.3, f"8b batch16 trees {trees}")


def test_sample_duplicate_siblings_rejected():
    """Two children of one node with the same token: the tree is refused on the device
    (status EAGLE_ERR_TREE), that sequence gets accept_len -1 and nothing is committed."""
    wl = _mini(seed=9)
    ref_tokens = wl.tokens.copy()
    par = wl.parents[0]
    kids = [j for j in range(1, len(par)) if par[j] == 0]
    ref_tokens[kids[1]] = ref_tokens[kids[0]]
    import torch
    from tree_attention_verification_06_amd.runner import TreeVerifier
    from workloads.device import to_tensor, upload
    t = upload(wl)
    M = wl.n_nodes
    gumbel, u = sample_inputs(wl, 2)
    v = TreeVerifier(wl.dims, t["weights"], t["k_cache"], t["v_cache"], batch=wl.batch, max_total_nodes=M,
                     max_nodes=max(len(p) for p in wl.parents), max_prefix=int(wl.prefix_len.max()), sample=True)
    t_tok = to_tensor(ref_tokens, "cuda")
    kc0 = np_of(t["k_cache"]).copy()
    v.step_sample(t["tree_off"], t["parent"], t_tok, t["prefix_len"], M, 1.0, to_tensor(gumbel, "cuda"),
                  to_tensor(u, "cuda"), x=t["x"])
    torch.cuda.synchronize()
    assert int(v.status.item()) == EAGLE_ERR_TREE
    assert int(v.accept_len[0].item()) == -1 and int(v.next_token[0].item()) == -1
    assert (np_of(v.path)[0] == -1).all()
    assert int(t["prefix_len"][0].item()) == int(wl.prefix_len[0])
    assert np.array_equal(np_of(t["k_cache"])[0], kc0[0])
    # the other sequences are accepted as usual
    assert (np_of(v.accept_len)[1:] >= 0).all()


def test_sample_distribution_tiny_fp32():
    """Distribution equality on the GPU path itself: many steps on one tree with fresh noise
    rows and uniforms each; the first emitted token follows the target's softmax(z_root)
    (children planted as the root's top tokens, so both acceptance and the bonus draw
    contribute), and the token after an accepted child follows softmax(z_child)."""
    import torch
    from tree_attention_verification_06_amd.runner import TreeVerifier
    from workloads.device import to_tensor, upload
    T_ = 0.05
    wl = make_workload(1)
    ref = oracle_verify(wl, want_logits=True)
    logits = ref["logits"]
    tokens = _plant(wl, logits, np.random.default_rng(3))
    par = wl.parents[0]
    n, V = len(par), wl.dims.vocab
    t = upload(wl)
    v = TreeVerifier(wl.dims, t["weights"], t["k_cache"], t["v_cache"], batch=1, max_total_nodes=n, max_nodes=n,
                     max_prefix=int(wl.prefix_len.max()), sample=True)
    trials = 3000
    rng = np.random.default_rng(17)
    U = rng.random((trials, V))
    g_all = to_tensor((-np.log(-np.log(np.where(U > 0, U, 1e-300)))).astype(np.float32), "cuda")
    u_all = to_tensor(rng.random((trials, n)).astype(np.float32), "cuda")
    t_tok = to_tensor(tokens, "cuda")
    p0 = t["prefix_len"].clone()
    outs = torch.zeros(trials, 2, dtype=torch.int32, device="cuda")
    lens = torch.zeros(trials, dtype=torch.int32, device="cuda")
    v.encode(t["tree_off"], t["parent"], t["prefix_len"], n)
    for i in range(trials):
        t["prefix_len"].copy_(p0)
        v.verify_sample(t["tree_off"], t_tok, t["parent"], t["prefix_len"], n, T_, g_all[i], x=t["x"])
        v.accept_sample(t["tree_off"], t["parent"], t_tok, u_all[i], t["prefix_len"])
        outs[i] = v.out_tokens[0, :2]
        lens[i] = v.accept_len[0]
    torch.cuda.synchronize()
    assert int(v.status.item()) == 0
    outs, lens = outs.cpu().numpy(), lens.cpu().numpy()

    def softmax(z):
        e = np.exp(z - z.max())
        return e / e.sum()

    def check(samples, p, label):
        # buckets: the 8 most likely tokens, then everything else
        top = np.argsort(-p)[:8]
        freq = np.array([(samples == k).mean() for k in top] + [(~np.isin(samples, top)).mean()])
        pb = np.concatenate([p[top], [1.0 - p[top].sum()]])
        bound = 5.0 * np.sqrt(pb * (1 - pb) / len(samples)) + 2e-3
        _log(label, "n", len(samples), "p", np.round(pb, 3).tolist(), "freq", np.round(freq, 3).tolist())
        assert np.all(np.abs(freq - pb) <= bound), (label, freq, pb)

    check(outs[:, 0], softmax(logits[0] / T_), "first token")
    kids = [c for c in range(1, n) if par[c] == 0]
    c_best = max(kids, key=lambda c: (outs[:, 0] == tokens[c]).sum())
    sel = (outs[:, 0] == tokens[c_best]) & (lens >= 1)
    assert sel.sum() >= 300, sel.sum()
    check(outs[sel, 1], softmax(logits[c_best] / T_), f"after child {c_best}")
