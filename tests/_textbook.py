"""Textbook sequential (causal, one token at a time) decoding, written independently of ``oracle/``.

Used only to pin the oracle: tree verification must reproduce exactly what a
plain left-to-right decoder computes ("Speculative decoding with EAGLE" page:
the output is identical to what the target produces alone).  Rotary
embedding here uses the complex-number form (pair (j, j + D/2) as the complex
number x_j + i x_{j+D/2}, multiplied by exp(i * pos * theta^(-2j/D))), and
attention is an explicit loop over past positions, so a slip in the oracle's
vectorised forms would show up as a mismatch.
"""
import math

import numpy as np


def wf(a):
    from workloads.bf16 import bf16_bits_to_f64
    a = np.asarray(a)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def rope_complex(vec, pos, theta):
    """vec [heads][D] rotated to position pos."""
    D = vec.shape[-1]
    half = D // 2
    z = vec[..., :half] + 1j * vec[..., half:]
    ang = np.array([pos * theta ** (-(2.0 * j) / D) for j in range(half)])
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def rmsnorm(v, gain, eps):
    return v / math.sqrt(float(np.dot(v, v)) / v.size + eps) * wf(gain)


class SequentialDecoder:
    """One decoder layer with a growing KV cache; step() consumes one token's input vector."""

    def __init__(self, dims, w, k_prefix=None, v_prefix=None):
        self.d = dims
        self.w = {k: wf(v) for k, v in w.items() if k not in ("embed", "w_lm", "final_ln", "w_fc")}
        Hkv, D = dims.n_kv_heads, dims.head_dim
        self.K = [] if k_prefix is None else [wf(k_prefix[:, t]) for t in range(k_prefix.shape[1])]
        self.V = [] if v_prefix is None else [wf(v_prefix[:, t]) for t in range(v_prefix.shape[1])]

    @property
    def pos(self):
        return len(self.K)

    def step(self, x):
        d, w = self.d, self.w
        H, D, Hq, Hkv = d.hidden, d.head_dim, d.n_q_heads, d.n_kv_heads
        g = Hq // Hkv
        norm = d.rms_eps > 0
        xh = rmsnorm(x, w["ln_attn"], d.rms_eps) if norm else x
        qkv = w["w_qkv"] @ xh
        q = qkv[: Hq * D].reshape(Hq, D)
        k = qkv[Hq * D: (Hq + Hkv) * D].reshape(Hkv, D)
        v = qkv[(Hq + Hkv) * D:].reshape(Hkv, D)
        p = self.pos
        if d.rope_theta > 0:
            q = rope_complex(q, p, d.rope_theta)
            k = rope_complex(k, p, d.rope_theta)
        self.K.append(k)
        self.V.append(v)
        o = np.zeros((Hq, D))
        for h in range(Hq):
            kvh = h // g
            scores = [float(np.dot(q[h], kk[kvh])) / math.sqrt(D) for kk in self.K]
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            tot = sum(ws)
            for wt, vv in zip(ws, self.V):
                o[h] += (wt / tot) * vv[kvh]
        y = x + w["w_o"] @ o.reshape(-1)
        if d.ffn > 0:
            yh = rmsnorm(y, w["ln_mlp"], d.rms_eps)
            gt = w["w_gate"] @ yh
            up = w["w_up"] @ yh
            a = gt / (1.0 + np.exp(-gt)) * up
            out = y + w["w_down"] @ a
        else:
            out = y
        return dict(q=q, k=k, v=v, attn=o.reshape(-1), h=out)


def logits_of(dims, weights, h):
    hn = rmsnorm(h, weights["final_ln"], dims.rms_eps) if dims.rms_eps > 0 else h
    return wf(weights["w_lm"]) @ hn


def greedy(z):
    """First index of the maximum, by an explicit scan."""
    best = 0
    for i in range(1, len(z)):
        if z[i] > z[best]:
            best = i
    return best
