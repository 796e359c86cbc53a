"""Pins of the oracle's acceptance at temperature T > 0 (oracle.sample_accept_sequence):
the emitted tokens follow the target's own distribution at every position (statistically,
with fresh random inputs per trial), the T -> 0 limit is the greedy rule (pinned on its own),
and a rejected child's token is never drawn as the bonus."""
import numpy as np

import oracle
from oracle.tree import tree_encode


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _gumbel(rng, shape):
    return -np.log(-np.log(rng.random(shape)))


def _trials(parent, tokens, logits, T, n, seed):
    rng = np.random.default_rng(seed)
    outs = []
    for _ in range(n):
        u = rng.random(len(parent))
        g = _gumbel(rng, logits.shape)
        outs.append(oracle.sample_accept_sequence(parent, tokens, logits, T, u, g)[2])
    return outs


def _check_freq(samples, p, n_min=2000):
    samples = np.asarray(samples)
    assert len(samples) >= n_min
    freq = np.bincount(samples, minlength=len(p)) / len(samples)
    bound = 5.0 * np.sqrt(p * (1 - p) / len(samples)) + 1e-3
    assert np.all(np.abs(freq - p) <= bound), (freq, p)


def test_emitted_tokens_follow_the_target_distribution():
    V, T = 6, 0.8
    # root -> children 1, 2, 3 (tokens 0, 2, 4); node 1 -> children 4, 5 (tokens 1, 3)
    parent = [-1, 0, 0, 0, 1, 1]
    tokens = [5, 0, 2, 4, 1, 3]
    logits = np.random.default_rng(0).normal(0.0, 1.0, (len(parent), V))
    outs = _trials(parent, tokens, logits, T, 60000, 1)
    # first emitted token ~ p(root), whether it came from an accepted child or the bonus
    _check_freq([o[0] for o in outs], _softmax(logits[0] / T))
    # second token given first = 0 (child 1 accepted) ~ p(node 1); given first = 2
    # (child 2 accepted, a leaf) it is the bonus ~ p(node 2)
    _check_freq([o[1] for o in outs if o[0] == 0], _softmax(logits[1] / T))
    _check_freq([o[1] for o in outs if o[0] == 2], _softmax(logits[2] / T), n_min=1000)


def test_low_temperature_is_the_greedy_rule():
    rng = np.random.default_rng(5)
    V = 50
    for trial in range(20):
        n = 12
        parent = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        logits = rng.normal(0.0, 1.0, (n, V))
        g = logits.argmax(axis=1)
        # tokens: half the children copy the parent's argmax, so paths get accepted
        tokens = [0] + [int(g[parent[j]]) if rng.random() < 0.5 else int(rng.integers(0, V)) for j in range(1, n)]
        for j in range(1, n):  # distinct sibling tokens
            sib = [i for i in range(1, j) if parent[i] == parent[j]]
            while tokens[j] in [tokens[i] for i in sib]:
                tokens[j] = int(rng.integers(0, V))
        enc = tree_encode(parent, 0)
        greedy = oracle.accept_sequence(parent, tokens, g, enc.depth)
        u = rng.uniform(1e-6, 1.0 - 1e-6, n)
        samp = oracle.sample_accept_sequence(parent, tokens, logits, 1e-4, u, _gumbel(rng, (n, V)))
        assert samp[0] == greedy[0] and samp[2] == greedy[2], (trial, samp, greedy)


def test_rejected_tokens_are_never_the_bonus():
    V = 8
    parent = [-1, 0, 0, 0]
    tokens = [7, 1, 2, 3]
    logits = np.random.default_rng(2).normal(0.0, 1.0, (4, V))
    rng = np.random.default_rng(3)
    for _ in range(500):
        u = np.ones(4)  # u * r < p(x) never holds: every child is rejected
        out = oracle.sample_accept_sequence(parent, tokens, logits, 1.0, u, _gumbel(rng, (4, V)))
        assert out[0] == 0 and out[2][0] not in (1, 2, 3)


def test_one_noise_row_per_tree_keeps_the_distribution():
    """The bonus is drawn once per walk, at a node that depends on u only, so one noise row
    shared by every node of the tree leaves each emitted token's distribution unchanged."""
    V, T = 6, 0.8
    parent = [-1, 0, 0, 0, 1, 1]
    tokens = [5, 0, 2, 4, 1, 3]
    logits = np.random.default_rng(0).normal(0.0, 1.0, (len(parent), V))
    rng = np.random.default_rng(11)
    outs = []
    for _ in range(60000):
        u = rng.random(len(parent))
        g = np.broadcast_to(_gumbel(rng, (V,)), logits.shape)
        outs.append(oracle.sample_accept_sequence(parent, tokens, logits, T, u, g)[2])
    _check_freq([o[0] for o in outs], _softmax(logits[0] / T))
    _check_freq([o[1] for o in outs if o[0] == 0], _softmax(logits[1] / T))
    _check_freq([o[1] for o in outs if o[0] == 2], _softmax(logits[2] / T), n_min=1000)


def _random_tree(rng, n, V):
    parent = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
    tokens = [int(rng.integers(0, V))]
    for j in range(1, n):
        sib = {tokens[i] for i in range(1, j) if parent[i] == parent[j]}
        t = int(rng.integers(0, V))
        while t in sib:
            t = int(rng.integers(0, V))
        tokens.append(t)
    return parent, tokens


def test_summaries_split_the_normaliser_and_exclude_children():
    """logsumexp(rest_lse[n], children's child_logit) is the full log-normaliser of z[n]
    (closed form: the vocabulary is the disjoint union of n's child tokens and the rest);
    child_logit is the tempered logit; rest_token is the noisy argmax over the rest, which is
    the plain noisy argmax whenever that is not a child token."""
    rng = np.random.default_rng(21)
    for trial in range(30):
        n, V, T = int(rng.integers(1, 15)), 40, float(rng.uniform(0.3, 2.0))
        parent, tokens = _random_tree(rng, n, V)
        logits = rng.normal(0.0, 2.0, (n, V))
        g = _gumbel(rng, (V,))
        cl, rl, rt = oracle.sample_summaries(parent, tokens, logits, T, g)
        z = logits / T
        for node in range(n):
            kids = [c for c in range(1, n) if parent[c] == node]
            for c in kids:
                assert cl[c] == z[node, tokens[c]]
            terms = np.array([rl[node]] + [cl[c] for c in kids])
            full = z[node].max() + np.log(np.exp(z[node] - z[node].max()).sum())
            assert abs((terms.max() + np.log(np.exp(terms - terms.max()).sum())) - full) < 1e-12
            assert rt[node] not in [tokens[c] for c in kids]
            plain = int(np.argmax(z[node] + g))
            if plain not in [tokens[c] for c in kids]:
                assert rt[node] == plain
        assert np.isnan(cl[0])


def test_summary_walk_is_the_full_walk():
    """The walk on the summaries takes the same decisions as the walk on the full logits with
    the tree's noise row at every node: same path, tokens, bonus and decision trace."""
    rng = np.random.default_rng(31)
    for trial in range(200):
        n, V = int(rng.integers(1, 20)), 30
        T = float(rng.choice([0.05, 0.3, 1.0]))
        parent, tokens = _random_tree(rng, n, V)
        logits = rng.normal(0.0, 1.0, (n, V))
        # make some children likely, so that walks go deep
        for c in range(1, n):
            if rng.random() < 0.5:
                logits[parent[c], tokens[c]] += 3.0
        g = _gumbel(rng, (V,))
        u = rng.random(n)
        t_full, t_sum = [], []
        full = oracle.sample_accept_sequence(parent, tokens, logits, T, u, np.broadcast_to(g, (n, V)), trace=t_full)
        cl, rl, rt = oracle.sample_summaries(parent, tokens, logits, T, g)
        summ = oracle.sample_accept_from_summaries(parent, tokens, cl, rl, rt, u, trace=t_sum)
        assert full[1] == summ[1] and full[2] == summ[2] and full[0] == summ[0], (trial, full, summ)
        assert [c for c, _, _ in t_full] == [c for c, _, _ in t_sum]
        assert np.allclose([p for _, _, p in t_full], [p for _, _, p in t_sum], rtol=1e-12, atol=0)


def test_duplicate_sibling_tokens_are_rejected():
    import pytest
    with pytest.raises(ValueError):
        oracle.sample_summaries([-1, 0, 0], [1, 2, 2], np.zeros((3, 5)), 1.0, np.zeros(5))
