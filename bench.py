#!/usr/bin/env python3
"""Benchmark of the EAGLE tree-verification step on one MI355X.

One step = eagle_tree_build + eagle_tree_verify + eagle_accept_commit over one batch of
synthetic trees (the whole verification hot path) on the seeded random-init workload of a
configuration; the headline is the Llama-3-8B-shaped layer with one 60-node static tree and
a 2048-token prefix.  The step is captured once into a HIP graph and replayed (its eager
launch sequence is timed too); each timed step sits between two HIP events, and the mean,
median and p90 of the step times are reported.  Prints one JSON line:
  value          = tree-verify nodes/s of the headline configuration (nodes / mean step time)
  accepted_tok_s = accepted tokens (L + 1 per sequence) per second, measured
  roofline       = the dominant kernel (LM head + fused argmax): algorithmic bytes per launch
                   / its mean launch time from HIP events recorded in the timed region
  step_roofline  = the step: sum over its kernels of max(bytes / 8 TB/s, flops / 2.5 PFLOP/s)
                   against the measured step time
  configs        = the same measurements for the other single-layer configurations (the tiny
                   fp32 layer, the ragged batch of four dynamic trees, the 70B-shaped layer
                   with a 32768-token prefix)
  eagle_step     = the full EAGLE step (draft + verify + accept) at batch 16
  cpu_baseline   = the fp64 CPU oracle on whole steps of the headline workload.
Inputs are resident in HBM before timing starts; the KV cache grows by the committed
tokens as a real decode loop does.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--other-configs", default="1,3,4",
                    help="single-layer configurations measured besides --config ('' for none)")
    ap.add_argument("--min-steps", type=int, default=50,
                    help="timed steps per configuration are max(--steps, this)")
    ap.add_argument("--no-graph", action="store_true", help="time the eager launch sequence only")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-nodes", type=int, default=0, help="0: one full step")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run a 1 GiB torch copy so counter runs can scale FETCH/WRITE_SIZE")
    ap.add_argument("--no-timer", action="store_true", help="time without per-kernel events")
    ap.add_argument("--no-eagle-step", action="store_true",
                    help="skip the full EAGLE step (draft + verify + accept, batch 16)")
    ap.add_argument("--eagle-steps", type=int, default=20)
    ap.add_argument("--weight-layout", choices=["packed", "row"], default="packed",
                    help="weight matrices (LM head, layer, draft): fragment-blocked (packed once at load) "
                         "or row-major")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="temperature of the sampling-acceptance measurements (T > 0)")
    ap.add_argument("--eagle-only", action="store_true",
                    help="run only the full EAGLE step (for profiling its kernels apart from the verify step)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-loop comparison over a stack of layers (EAGLE vs plain greedy)")
    ap.add_argument("--decode-only", action="store_true", help="run only the decode-loop comparison")
    ap.add_argument("--decode-layers", type=int, default=32,
                    help="target depth of the decode-loop comparison (32: the Llama-3-8B depth)")
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--decode-batches", default="1,16")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lm_head_bytes(dims, M):
    # weights once, the feature rows once (bf16 on the bf16 path), one packed key per row out
    es = 2 if dims.dtype == "bf16" else 4
    return dims.vocab * dims.hidden * es + M * dims.hidden * es + M * 8


def measured_traffic(workload_name, layout):
    """HBM bytes per LM-head launch from the committed counter summary, if it was taken on
    the GEMM source as it is now and with the same LM-head weight layout (None otherwise)."""
    import hashlib
    import glob
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    src = os.path.join(here, "tree_attention_verification_06_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if "8b-layer-60node" not in workload_name:
        return None
    for f in glob.glob(os.path.join(here, "profiles", "lm_head_hbm_traffic_*.md")):
        text = open(f).read()
        m1 = re.search(r"traffic_bytes_per_launch: (\d+)", text)
        m2 = re.search(r"gemm_source_sha256: ([0-9a-f]+)", text)
        m3 = re.search(r"weight_layout: (\S+)", text)
        if m1 and m2 and m3 and m2.group(1) == sha and m3.group(1) == layout:
            return int(m1.group(1))
    return None


def step_roofline_parts(dims, wl):
    """Algorithmic bytes and flops of each kernel of one verification step: every weight once,
    the KV prefix once, activations read once and written once (bf16 between GEMMs, the
    residual stream in fp32), tree K/V written once and read once; flops 2 per MAC over the
    real rows, attention 4 * Hq * D per visible key of each node (prefix + depth + 1)."""
    es = 2 if dims.dtype == "bf16" else 4
    H, Hq, Hkv, D, F, V = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab
    M = wl.n_nodes
    qkv = (Hq + 2 * Hkv) * D
    parts = {}
    parts["qkv"] = (qkv * H * es + M * H * es + M * qkv * es, 2 * M * qkv * H)
    att_flops = 0
    for b, par in enumerate(wl.parents):
        d = np.zeros(len(par), dtype=np.int64)
        for i in range(1, len(par)):
            d[i] = d[par[i]] + 1
        att_flops += int(np.sum(4 * Hq * D * (int(wl.prefix_len[b]) + d + 1)))
    kv = sum(int(p) for p in wl.prefix_len) * Hkv * D * 2 * es
    parts["attention"] = (kv + M * qkv * es + M * Hq * D * es, att_flops)
    parts["o_proj"] = (H * Hq * D * es + M * Hq * D * es + M * H * es + M * H * 4, 2 * M * H * Hq * D)
    if F > 0:
        parts["gate_up"] = (2 * F * H * es + M * H * es + M * F * es, 4 * M * F * H)
        parts["down"] = (F * H * es + M * F * es + M * H * 4 + M * H * 4, 2 * M * F * H)
    parts["lm_head"] = (V * H * es + M * H * es + M * 8, 2 * M * V * H)
    return parts


def step_roofline(dims, wl, ms_step):
    """T_roof = sum over kernels of max(bytes / HBM peak, flops / bf16 MFMA peak) (the fp32
    layer uses the fp32 vector peak, 157.3 TFLOP/s), against the measured step time."""
    peak_f = MFMA_BF16_PEAK_TFLOPS if dims.dtype == "bf16" else FP32_PEAK_TFLOPS
    parts = step_roofline_parts(dims, wl)
    kern = {}
    t_hbm = t_mfma = 0.0
    for k, (b, f) in parts.items():
        tb = b / (HBM_PEAK_GBS * 1e9) * 1e3
        tf = f / (peak_f * 1e12) * 1e3
        kern[k] = {"bytes": int(b), "flops": int(f), "bound": "hbm" if tb >= tf else "mfma",
                   "t_roof_ms": round(max(tb, tf), 6)}
        if tb >= tf:
            t_hbm += tb
        else:
            t_mfma += tf
    t_roof = t_hbm + t_mfma
    return {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "algorithmic_bytes": int(sum(b for b, _ in parts.values())),
            "algorithmic_flops": int(sum(f for _, f in parts.values())),
            "t_roof_ms": round(t_roof, 5), "t_roof_hbm_ms": round(t_hbm, 5), "t_roof_mfma_ms": round(t_mfma, 5),
            "frac": round(t_roof / ms_step, 4), "kernels": kern}


def draft_roofline_bytes_flops(dims, p, batch, prefix_len):
    """Algorithmic bytes and flops of one draft expansion: every level streams the FC, the
    draft layer and the LM head once and reads the draft KV prefix once; rows per level are
    B on the first level and B * frontier after it."""
    H, Hq, Hkv, D, F, V = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab
    w = 2 * H * H + (Hq + 2 * Hkv) * D * H + H * Hq * D + 3 * F * H + V * H
    kv = int(np.sum(prefix_len)) * Hkv * D * 2 * 2
    byts = p.depth * (w * 2 + kv)
    rows = batch + (p.depth - 1) * batch * p.frontier
    flops = 2 * rows * w + rows * 4 * Hq * D * (int(np.mean(prefix_len)) + p.depth)
    return byts, flops


def layout_name(args):
    return "fragment-blocked" if args.weight_layout == "packed" else "row-major"


def laid_out(weights, args):
    """The weights with every matrix in the layout --weight-layout asks for (packing is a
    load-time step, outside every timed region), and the layout code for the runners."""
    if args.weight_layout == "row":
        return weights, 0
    from tree_attention_verification_06_amd.runner import with_packed_weights
    return with_packed_weights(weights), 1


def bench_eagle_step(args):
    """The full speculative step at the 8B shape with batch 16 (draft -> tree build -> verify
    of the 16 x 60 drafted nodes -> accept + commit), as a decode loop: each step's roots are
    the previous step's bonus tokens and their features.  All on device, no host sync."""
    import torch
    import tree_attention_verification_06_amd as E
    from tree_attention_verification_06_amd.runner import EagleStep
    from workloads import make_workload
    from workloads.device import upload

    n = args.eagle_steps
    t0 = time.perf_counter()
    wl = make_workload(5, seed=args.seed, cache_slack=(n + 8) * 8)
    log(f"workload {wl.name}: generated in {time.perf_counter() - t0:.1f}s")
    t = upload(wl)
    dims, p, B = wl.dims, wl.draft, wl.batch
    weights, layout = laid_out(t["weights"], args)
    draft_weights, _ = laid_out(t["draft_weights"], args)
    st = EagleStep(dims, p, weights, draft_weights, t["k_cache"], t["v_cache"], t["dk_cache"],
                   t["dv_cache"], batch=B, max_prefix=wl.cache_cap, lm_layout=layout, weight_layout=layout,
                   sample=True)
    d, v = st.drafter, st.verifier
    prefix0 = t["prefix_len"].clone()
    feat = t["root_feature"].clone()
    tok = t["root_token"].clone()

    def run_steps(k, timer=None, count=False):
        nonlocal feat, tok
        acc = []
        for _ in range(k):
            nf, nt = st.step(feat, tok, t["prefix_len"], timer=timer)
            feat = nf.clone()
            tok = nt.clone()
            if count:
                acc.append(int((v.accept_len + 1).sum().item()))
        return acc

    run_steps(3)
    t["prefix_len"].copy_(prefix0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run_steps(n)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / n
    st_code = int(v.status.item())
    if st_code != 0:
        raise RuntimeError(f"device status {st_code} ({E.status_str(st_code)})")
    # the draft alone and the verification alone (same trees), same stream, no sync inside
    e0.record(stream)
    for _ in range(n):
        d.expand(feat, tok, t["prefix_len"])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_draft = e0.elapsed_time(e1) / n
    tokens_fixed = d.tokens.clone()
    plen = t["prefix_len"].clone()
    e0.record(stream)
    for _ in range(n):
        v.encode(d.tree_off, d.parent, plen, st.total)
        v.verify(d.tree_off, tokens_fixed, plen, st.total)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_verify = e0.elapsed_time(e1) / n
    # accepted tokens per step (a separate pass that reads accept_len after each step)
    t["prefix_len"].copy_(prefix0)
    acc = run_steps(min(n, 10), count=True)
    # per-stage breakdown of one draft expansion (diagnostic: events around every kernel)
    diag = E.Timer(capacity=4096)
    for _ in range(3):
        d.expand(feat, tok, t["prefix_len"], timer=diag)
    torch.cuda.synchronize()
    stages = {k: round(ms / 3, 5) for k, (ms, c) in diag.collect().items()}
    diag.close()
    dbytes, dflops = draft_roofline_bytes_flops(dims, p, B, wl.prefix_len)
    d_roof_ms = max(dbytes / (HBM_PEAK_GBS * 1e9), dflops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    eagle3 = bench_eagle3(args, wl, st, t, prefix0, feat, tok)
    sampling = bench_sampling(args, wl, st, t, prefix0, feat, tok)
    nodes = B * p.max_nodes
    acc_mean = float(np.mean(acc))
    return {
        "workload": wl.name, "batch": B, "prefix": int(wl.prefix_len.max()),
        "weight_layout": layout_name(args),
        "draft": {"depth": p.depth, "top_k": p.top_k, "frontier": p.frontier, "max_nodes": p.max_nodes,
                  "conf_threshold": p.conf_threshold},
        "steps": n, "ms_per_step": round(ms_step, 4), "ms_draft": round(ms_draft, 4),
        "ms_verify": round(ms_verify, 4),
        "accepted_per_step": acc_mean, "accepted_tok_s": round(acc_mean / (ms_step * 1e-3), 1),
        "verify_nodes_s": round(nodes / (ms_verify * 1e-3), 1),
        "draft_roofline": {"bound": "hbm", "algorithmic_bytes": dbytes, "algorithmic_flops": dflops,
                           "t_roof_ms": round(d_roof_ms, 4), "frac": round(d_roof_ms / ms_draft, 4)},
        "draft_stage_ms": stages,
        "eagle3": eagle3,
        "sampling": sampling,
        "data": "synthetic: random-init draft head and target layer N(0,0.02), root features N(0,1), "
                "draft KV prefix N(0,1); the roots of each step are the previous step's bonus tokens",
    }


def layer_bytes(dims):
    """Weight bytes of one bf16 decoder layer (QKV, O, gate, up, down; gains ignored)."""
    H, D, Hq, Hkv, F = dims.hidden, dims.head_dim, dims.n_q_heads, dims.n_kv_heads, dims.ffn
    return 2 * (dims.qkv_rows * H + H * Hq * D + 3 * F * H)


def bench_decode(args):
    """A target of --decode-layers Llama-3-8B-shaped layers under the shared LM head, with a
    2048-token prefix, decoded two ways through the same kernels at each batch of
    --decode-batches:
      plain greedy decoding: the one-node tree of each sequence's last token per step
        (tree build -> verify through every layer -> accept + commit = the argmax);
      EAGLE: draft (depth 6, top-10, frontier 10, 60 nodes) -> tree build -> verify of the
        drafted nodes through every layer -> accept + commit every layer -> draft KV update
        of the committed positions from the target's true features.
    Both loops run on device without host synchronisation; the cache grows by the committed
    tokens.  With random weights the drafts are not accepted (L = 0), so the measured
    speedup is that of one token per step; the break-even accepted length and the speedup
    projected at 3.5 and 4.5 tokens per step (the pages' typical accepted lengths) follow
    from the two step times.  Weights and caches are drawn on the device with torch's
    generator (N(0, 0.02) weights, N(0, 1) caches and features): the stack is 14 GB."""
    import torch
    import tree_attention_verification_06_amd as E
    from tree_attention_verification_06_amd.runner import EagleStackStep, GreedyStackDecoder, with_packed_weights
    from workloads import DraftParams
    from workloads.configs import LLAMA8B

    dims, nl, n = LLAMA8B, args.decode_layers, args.decode_steps
    H, D, Hq, Hkv, F, V = dims.hidden, dims.head_dim, dims.n_q_heads, dims.n_kv_heads, dims.ffn, dims.vocab
    p = DraftParams()
    packed = args.weight_layout == "packed"
    layout = 1 if packed else 0
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5000 if args.seed is None else args.seed)

    def randn(*shape, std=0.02):
        x = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
        x.normal_(0.0, std, generator=gen)
        return x

    def ones():
        return torch.ones(H, dtype=torch.bfloat16, device="cuda")

    def layer():
        w = dict(ln_attn=ones(), ln_mlp=ones(), w_qkv=randn(dims.qkv_rows, H), w_o=randn(H, Hq * D),
                 w_gate=randn(F, H), w_up=randn(F, H), w_down=randn(H, F))
        return with_packed_weights(w, lm_head=False) if packed else w

    t0 = time.perf_counter()
    layers = [layer() for _ in range(nl)]
    head = dict(final_ln=ones(), w_lm=randn(V, H), embed=randn(V, H))
    if packed:
        head = with_packed_weights(head, layer=False)
    dw = layer()
    dw["w_fc"] = E.eagle_pack_fragments(randn(H, 2 * H)) if packed else randn(H, 2 * H)
    torch.cuda.synchronize()
    log(f"decode: {nl} layers drawn and laid out in {time.perf_counter() - t0:.1f}s")
    P0 = 2048
    warm = 3
    cap = P0 + (warm + 2 * n + 4) * (p.depth + 1) + 16
    stack_bytes = nl * layer_bytes(dims) + lm_head_bytes(dims, 1)
    out = {"target": f"{nl} Llama-3-8B-shaped decoder layers + LM head (vocab {V})", "n_layers": nl,
           "prefix": P0, "weight_layout": layout_name(args), "steps": n,
           "draft": {"depth": p.depth, "top_k": p.top_k, "frontier": p.frontier, "max_nodes": p.max_nodes,
                     "conf_threshold": p.conf_threshold},
           "batches": {}}
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    def run_loops(B, kc, vc, dkc, dvc, root_tok, root_feat, count):
        """ms per step of plain greedy decoding and of the EAGLE step on the given caches (and
        the emitted tokens per step of the EAGLE loop when ``count``)."""
        prefix = torch.full((B,), P0, dtype=torch.int32, device="cuda")
        dec = GreedyStackDecoder(dims, head, layers, kc, vc, batch=B, max_prefix=cap, lm_layout=layout,
                                 weight_layout=layout)
        tok = root_tok.clone()
        for _ in range(warm):
            tok = dec.step(tok, prefix).clone()
        prefix.fill_(P0)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            tok = dec.step(tok, prefix)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_plain = e0.elapsed_time(e1) / n
        if int(dec.v.status.item()) != 0:
            raise RuntimeError(f"plain decode: device status {int(dec.v.status.item())}")
        del dec
        st = EagleStackStep(dims, p, head, layers, dw, kc, vc, dkc, dvc, batch=B, max_prefix=cap, lm_layout=layout,
                            weight_layout=layout)
        prefix.fill_(P0)
        feat, tok = root_feat.clone(), root_tok.clone()
        for _ in range(warm):
            feat, tok = st.step(feat, tok, prefix)
        prefix.fill_(P0)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            feat, tok = st.step(feat, tok, prefix)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_eagle = e0.elapsed_time(e1) / n
        acc = []  # emitted tokens per step (a separate pass that reads accept_len after each step)
        for _ in range(n if count else 0):
            feat, tok = st.step(feat, tok, prefix)
            acc.append(int((st.verifier.accept_len + 1).sum().item()))
        if int(st.verifier.status.item()) != 0:
            raise RuntimeError(f"EAGLE decode: device status {int(st.verifier.status.item())}")
        del st
        return ms_plain, ms_eagle, acc

    PSZ = 64
    for B in [int(b) for b in args.decode_batches.split(",") if b]:
        root_tok = torch.randint(0, V, (B,), dtype=torch.int32, device="cuda", generator=gen)
        root_feat = torch.empty(B, H, dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=gen)
        kc = randn(nl, B, Hkv, cap, D, std=1.0)
        vc = randn(nl, B, Hkv, cap, D, std=1.0)
        dkc = randn(B, Hkv, cap, D, std=1.0)
        dvc = randn(B, Hkv, cap, D, std=1.0)
        ms_plain, ms_eagle, acc = run_loops(B, kc, vc, dkc, dvc, root_tok, root_feat, True)
        del kc, vc, dkc, dvc
        torch.cuda.empty_cache()
        # the same loops on paged caches: 64-token pages, every sequence's pages scattered
        # over the pool by a random permutation (the continuous-batching layout)
        maxb = -(-cap // PSZ)
        n_pages = B * maxb
        perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(B)).to(torch.int32)
        table = perm.reshape(B, maxb).to("cuda")
        kp = E.PagedCache(randn(nl, n_pages, Hkv, PSZ, D, std=1.0), table, PSZ)
        vp = E.PagedCache(randn(nl, n_pages, Hkv, PSZ, D, std=1.0), table, PSZ)
        dkp = E.PagedCache(randn(n_pages, Hkv, PSZ, D, std=1.0), table, PSZ)
        dvp = E.PagedCache(randn(n_pages, Hkv, PSZ, D, std=1.0), table, PSZ)
        pms_plain, pms_eagle, _ = run_loops(B, kp, vp, dkp, dvp, root_tok, root_feat, False)
        del kp, vp, dkp, dvp
        torch.cuda.empty_cache()
        acc_seq = float(np.mean(acc)) / B  # emitted tokens per sequence per step
        kv_bytes = nl * B * Hkv * P0 * D * 2 * 2
        roof_plain_ms = (stack_bytes + kv_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3
        out["batches"][str(B)] = {
            "plain_ms_per_step": round(ms_plain, 4), "plain_tok_s": round(B / (ms_plain * 1e-3), 1),
            "plain_roofline": {"bound": "hbm", "algorithmic_bytes": stack_bytes + kv_bytes,
                               "t_roof_ms": round(roof_plain_ms, 4), "frac": round(roof_plain_ms / ms_plain, 4)},
            "eagle_ms_per_step": round(ms_eagle, 4), "eagle_tokens_per_seq_step": round(acc_seq, 3),
            "eagle_tok_s": round(acc_seq * B / (ms_eagle * 1e-3), 1),
            "speedup_measured": round(acc_seq * ms_plain / ms_eagle, 3),
            "break_even_tokens_per_step": round(ms_eagle / ms_plain, 3),
            "projected_speedup": {str(tau): round(tau * ms_plain / ms_eagle, 3) for tau in (3.5, 4.5)},
            "paged": {"page_size": PSZ, "plain_ms_per_step": round(pms_plain, 4),
                      "eagle_ms_per_step": round(pms_eagle, 4),
                      "plain_overhead_pct": round(100 * (pms_plain / ms_plain - 1), 2),
                      "eagle_overhead_pct": round(100 * (pms_eagle / ms_eagle - 1), 2)},
        }
        log(f"decode B={B}: plain {ms_plain:.3f} ms/step (paged {pms_plain:.3f}), EAGLE {ms_eagle:.3f} ms/step "
            f"(paged {pms_eagle:.3f}), {acc_seq:.2f} tokens/seq/step")
    out["data"] = ("synthetic: random-init target stack, LM head, embedding and draft head N(0,0.02) drawn on the "
                   "device; KV prefixes and root features N(0,1); each step's roots are the previous step's bonus "
                   "tokens")
    return out


def bench_sampling(args, wl, st, t, prefix0, feat, tok):
    """Acceptance at temperature T > 0 at the same shape (16 trees of up to 60 drafted nodes):
    the sampling verification alone (encode + eagle_tree_verify_sample on fixed drafted trees;
    its LM head reads one noise row of V floats per tree on top of the weights) and whole
    sampling steps (draft -> encode -> verify_sample -> accept_sample, decode loop).  The
    noise rows and acceptance uniforms are seeded inputs, resident before the timed region
    and reused by every step."""
    import torch
    import tree_attention_verification_06_amd as E
    from workloads.configs import sample_inputs

    n = args.eagle_steps
    T = args.temperature
    d, v = st.drafter, st.verifier
    gumbel, u = sample_inputs(wl, 0, n_nodes=st.total)
    g_t = torch.from_numpy(gumbel).cuda()
    u_t = torch.from_numpy(u).cuda()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # verification alone, on the trees of one draft expansion
    t["prefix_len"].copy_(prefix0)
    d.expand(feat, tok, t["prefix_len"])
    tokens_fixed = d.tokens.clone()
    plen = t["prefix_len"].clone()

    def verify_only(k, timer=None):
        for _ in range(k):
            v.encode(d.tree_off, d.parent, plen, st.total)
            v.verify_sample(d.tree_off, tokens_fixed, d.parent, plen, st.total, T, g_t, timer=timer)

    verify_only(3)
    torch.cuda.synchronize()
    lm = E.Timer(capacity=4 * (n + 1), stages=["lm_head"])
    e0.record(stream)
    verify_only(n, lm)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_verify = e0.elapsed_time(e1) / n
    lm_ms, lm_n = lm.collect().get("lm_head", (0.0, 0))
    lm.close()
    diag = E.Timer(capacity=64)
    verify_only(3, diag)
    torch.cuda.synchronize()
    stages = {k: round(ms / 3, 5) for k, (ms, c) in diag.collect().items()}
    diag.close()

    # whole sampling steps
    f, tk = feat.clone(), tok.clone()

    def run(k, count=False):
        nonlocal f, tk
        acc = []
        for _ in range(k):
            nf, nt = st.step_sample(f, tk, t["prefix_len"], T, g_t, u_t)
            f, tk = nf.clone(), nt.clone()
            if count:
                acc.append(int((v.accept_len + 1).sum().item()))
        return acc

    t["prefix_len"].copy_(prefix0)
    run(3)
    t["prefix_len"].copy_(prefix0)
    torch.cuda.synchronize()
    e0.record(stream)
    run(n)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / n
    st_code = int(v.status.item())
    if st_code != 0:
        raise RuntimeError(f"device status {st_code} ({E.status_str(st_code)})")
    t["prefix_len"].copy_(prefix0)
    acc = run(min(n, 10), count=True)
    acc_mean = float(np.mean(acc))
    nodes = st.total
    # the sampling LM head at 960 rows is bound by MFMA (2 M H V flops), not by its bytes
    # (weights once, bf16 feature rows, the noise rows, 12 bytes of results per row)
    dims = wl.dims
    lm_avg = lm_ms / max(lm_n, 1)
    flops = 2.0 * nodes * dims.hidden * dims.vocab
    byts = dims.vocab * dims.hidden * 2 + nodes * dims.hidden * 2 + gumbel.nbytes + nodes * 12
    lm_roof = None
    if lm_n:
        ach = flops / (lm_avg * 1e-3) / 1e12
        lm_roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
                   "algorithmic_bytes": byts,
                   "hbm_frac": round(byts / (lm_avg * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "kernel": "gemm_bf16_kernel<..., SAMPLE> (LM head + sampling epilogue)"}
    return {
        "temperature": T, "ms_verify": round(ms_verify, 4),
        "verify_nodes_s": round(nodes / (ms_verify * 1e-3), 1),
        "lm_head_ms": round(lm_avg, 4),
        "lm_head_roofline": lm_roof,
        "verify_stage_ms": stages,
        "ms_per_step": round(ms_step, 4),
        "accepted_per_step": acc_mean, "accepted_tok_s": round(acc_mean / (ms_step * 1e-3), 1),
        "noise_bytes_per_step": int(gumbel.nbytes),
        "data": "seeded Gumbel noise rows [B][V] and acceptance uniforms, fixed across steps",
    }


def bench_eagle3(args, wl, st, t, prefix0, feat, tok):
    """EAGLE-3 draft input at the same shape: the root features are W_fuse [f_low; f_mid; f_high]
    (eagle_fuse_features, K = 3H) instead of the top feature.  Times the fusion alone (HIP
    events around n launches; HBM roofline of its weight stream) and whole EAGLE-3 steps
    (fuse -> draft -> encode -> verify -> accept).  The one-layer target cannot produce three
    feature levels, so every step fuses the same seeded synthetic low/mid/high features."""
    import torch
    import tree_attention_verification_06_amd as E
    from workloads.configs import eagle3_inputs
    n = args.eagle_steps
    dims, B, H = wl.dims, wl.batch, wl.dims.hidden
    w_np, f_np = eagle3_inputs(wl)
    w_fuse = torch.from_numpy(w_np.view(np.int16)).cuda().view(torch.bfloat16)
    feats = torch.from_numpy(f_np.view(np.int16)).cuda().view(torch.bfloat16)
    layout = 1 if args.weight_layout == "packed" else 0
    if layout:
        w_fuse = E.eagle_pack_fragments(w_fuse)
    root = torch.zeros(B, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(E.eagle_workspace_size(2, dims, B, 0, 0, 0), dtype=torch.uint8, device="cuda")
    E.eagle_workspace_init(ws)

    def fuse():
        E.eagle_fuse_features(dims, w_fuse, feats, root, ws, w_layout=layout)
    for _ in range(3):
        fuse()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fuse()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_fuse = e0.elapsed_time(e1) / n
    t["prefix_len"].copy_(prefix0)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fuse()
        st.step(root, tok, t["prefix_len"])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / n
    fbytes = H * 3 * H * 2 + B * 3 * H * 2 + B * H * 4
    return {"fuse": f"W_fuse [{H}][{3 * H}] on [f_low; f_mid; f_high] of {B} sequences",
            "ms_fuse": round(ms_fuse, 4), "ms_per_step": round(ms_step, 4),
            "fuse_roofline": {"bound": "hbm", "algorithmic_bytes": fbytes,
                              "frac": round(fbytes / (ms_fuse * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}}


def cpu_baseline(wl, sample_nodes, min_seconds=10.0, max_steps=100):
    """The fp64 oracle (as it is) on the same workload, on this host's cores: whole
    verification steps (tree encode, layer forward, LM-head argmax, accept, commit)
    repeated until at least min_seconds of CPU work have been timed.  The commit writes into
    cache copies made once before the timed loop (each step commits the same slots)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    parents = wl.parents
    x = wl.x
    tokens = wl.tokens
    if sample_nodes:
        parents = [parents[0][:sample_nodes]]
        x = x[:sample_nodes]
        tokens = tokens[:sample_nodes]
    n = sum(len(p) for p in parents)
    kc = wl.k_cache.copy()
    vc = wl.v_cache.copy()
    steps = 0
    acc = 0
    t0 = time.perf_counter()
    while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        out = oracle.verify_forward(wl.dims, wl.weights, x, parents, wl.prefix_len[:len(parents)], wl.k_cache,
                                    wl.v_cache, want_logits=False)
        res = oracle.accept_batch(parents, tokens, out["argmax"], out["encs"])
        off = 0
        for b, (L, path, *_rest) in enumerate(res):
            oracle.commit_sequence(kc[b], vc[b], out["k_tree"][off:off + len(parents[b])],
                                   out["v_tree"][off:off + len(parents[b])], path, int(wl.prefix_len[b]))
            off += len(parents[b])
        acc += sum(r[0] + 1 for r in res)
        steps += 1
    dt = time.perf_counter() - t0
    return dict(value=n * steps / dt, unit="nodes/s", cores=threads, host_cores=host_cores,
                blas_threads=threads, kind="oracle",
                sample=f"{steps} full verification steps of the same workload ({n} nodes each: tree encode, "
                       f"fp64 layer forward, LM-head argmax, accept, commit into cache copies made once)",
                seconds=round(dt, 2), accepted_tok_s=acc / dt)


def _stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "min": round(float(a.min()), 5), "n": int(len(a))}


def _timed_steps(run_one, n, stream):
    """Per-step times (ms) of n steps, each between two HIP events on `stream`; returns the
    list and the time from the first event to the last."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        run_one()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)], ev[0].elapsed_time(ev[n])


def bench_verify(cfg, args, *, steps, warmup, headline=False):
    """Tree build + verify + accept/commit on configuration cfg: the eager launch sequence
    (with HIP events around the LM head for its per-launch roofline) and the same step
    captured once into a HIP graph and replayed; per-kernel diagnostic times; accepted
    tokens per step, measured and with one planted depth-3 path."""
    import torch
    import tree_attention_verification_06_amd as E
    from tree_attention_verification_06_amd.runner import TreeVerifier
    from workloads import make_workload, trees as T
    from workloads.device import upload

    n_stats = max(steps, args.min_steps)
    t0 = time.perf_counter()
    wl = make_workload(cfg, seed=args.seed, cache_slack=(max(warmup, n_stats) + 24) * 2)
    dims = wl.dims
    log(f"workload {wl.name}: {wl.n_nodes} nodes, batch {wl.batch}, generated in {time.perf_counter() - t0:.1f}s")
    t = upload(wl)
    torch.cuda.synchronize()
    M = wl.n_nodes
    max_nodes = max(len(p) for p in wl.parents)
    weights, layout = laid_out(t["weights"], args) if dims.dtype == "bf16" else (t["weights"], 0)
    v = TreeVerifier(dims, weights, t["k_cache"], t["v_cache"], batch=wl.batch, max_total_nodes=M,
                     max_nodes=max_nodes, max_prefix=int(wl.prefix_len.max()), lm_layout=layout,
                     weight_layout=layout)
    prefix0 = t["prefix_len"].clone()
    stream = torch.cuda.current_stream()

    def step(timer=None):
        v.step(t["tree_off"], t["parent"], t["tokens"], t["prefix_len"], M, x=t.get("x"), timer=timer)

    def check_status(where):
        st = int(v.status.item())
        if st != 0:
            raise RuntimeError(f"{wl.name} {where}: device status {st} ({E.status_str(st)})")

    for _ in range(warmup):
        step()
    t["prefix_len"].copy_(prefix0)
    # eager launches; HIP events around the dominant kernel (the LM head) only
    timer = None if args.no_timer else E.Timer(capacity=4 * (n_stats + 1), stages=["lm_head"])
    eager_ms, _ = _timed_steps(lambda: step(timer), n_stats, stream)
    stages = timer.collect() if timer else {}
    if timer:
        timer.close()
    check_status("eager")
    # the step as one HIP graph, replayed
    graph_ms = None
    g_total = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        t["prefix_len"].copy_(prefix0)
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            with torch.cuda.graph(graph, stream=cs):
                step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        t["prefix_len"].copy_(prefix0)
        graph_ms, g_total = _timed_steps(graph.replay, steps, stream)   # exactly `steps` timed steps
        stats_ms = graph_ms
        if n_stats > steps:
            t["prefix_len"].copy_(prefix0)
            stats_ms, _ = _timed_steps(graph.replay, n_stats, stream)
        check_status("graph")
        del graph
    # per-kernel breakdown: a separate pass with events around every kernel (diagnostic)
    t["prefix_len"].copy_(prefix0)
    diag = E.Timer(capacity=16 * 11)
    for _ in range(10):
        step(diag)
    torch.cuda.synchronize()
    diag_stages = diag.collect()
    diag.close()
    # accepted tokens per step: the same steps again, reading accept_len after each (untimed)
    t["prefix_len"].copy_(prefix0)
    accepted = []
    for _ in range(10):
        step()
        accepted.append(int((v.accept_len + 1).sum().item()))
    acc_per_step = float(np.mean(accepted))
    # planted variant: tokens along one depth-3 root path per tree set to the target's greedy
    # choice (node inputs are given hidden states, so tokens do not change the target's argmax)
    t["prefix_len"].copy_(prefix0)
    step()
    torch.cuda.synchronize()
    g = v.argmax.cpu().numpy()
    tokens = wl.tokens.copy()
    for b, par in enumerate(wl.parents):
        o = int(wl.tree_off[b])
        d = T.depths(par)
        cands = [i for i in range(len(par)) if d[i] == 3] or [max(range(len(par)), key=lambda i: d[i])]
        j = cands[0]
        while j > 0:
            tokens[o + j] = g[o + par[j]]
            j = par[j]
    t_tokens = torch.from_numpy(tokens).cuda()
    t["prefix_len"].copy_(prefix0)
    v.step(t["tree_off"], t["parent"], t_tokens, t["prefix_len"], M, x=t.get("x"))
    planted = int((v.accept_len + 1).sum().item())
    check_status("planted")

    timed = graph_ms if graph_ms is not None else eager_ms[:steps]
    ms_per_step = float(np.mean(timed))
    lm_ms, lm_n = stages.get("lm_head", (0.0, 0))
    roof = None
    if lm_n:
        lm_avg = lm_ms / lm_n
        ach = lm_head_bytes(dims, M) / (lm_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, layout_name(args)),
                "kernel": "gemm_bf16_kernel (LM head + fused row argmax)" if dims.dtype == "bf16" else
                "gemm_f32_kernel (LM head + fused row argmax)",
                "kernel_ms": round(lm_avg, 5), "bytes_per_launch": lm_head_bytes(dims, M),
                "flops_per_launch": 2 * M * dims.hidden * dims.vocab,
                "mfma_frac": round(2 * M * dims.hidden * dims.vocab / (lm_avg * 1e-3) / 1e12 /
                                   (MFMA_BF16_PEAK_TFLOPS if dims.dtype == "bf16" else FP32_PEAK_TFLOPS), 4)}
    out = {
        "workload": wl.name, "batch": wl.batch, "tree_nodes": M, "max_tree_nodes": max_nodes,
        "tree_sizes": [len(p) for p in wl.parents], "prefix": [int(p) for p in wl.prefix_len],
        "dtype": "bf16" if dims.dtype == "bf16" else "f32",
        "shape": {"hidden": dims.hidden, "q_heads": dims.n_q_heads, "kv_heads": dims.n_kv_heads,
                  "head_dim": dims.head_dim, "ffn": dims.ffn, "vocab": dims.vocab},
        "timed_steps": len(timed), "launch": "hip_graph" if graph_ms is not None else "eager",
        "ms_per_step": round(ms_per_step, 5), "us_per_step": round(ms_per_step * 1e3, 2),
        "step_ms": _stats(stats_ms if graph_ms is not None else eager_ms),
        "eager_step_ms": _stats(eager_ms),
        "nodes_s": round(M / (ms_per_step * 1e-3), 1),
        "accepted_per_step": acc_per_step,
        "accepted_tok_s": round(acc_per_step / (ms_per_step * 1e-3), 1),
        "accepted_tok_s_planted_depth3": round(planted / (ms_per_step * 1e-3), 1),
        "step_roofline": step_roofline(dims, wl, ms_per_step),
        "lm_head_roofline": roof,
        "stage_ms_per_step": {k: round(ms / max(n, 1), 5) for k, (ms, n) in diag_stages.items()},
    }
    if headline:
        out["_wl"] = wl
    del v, t
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the verification step runs on one MI355X; "
              f"no cross-GPU path is built); got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)
    import torch
    import tree_attention_verification_06_amd as E

    E.lib()  # fail loudly if the HIP library is not built
    if args.eagle_only:
        print(json.dumps({"eagle_step": bench_eagle_step(args)}), flush=True)
        return
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(args)}), flush=True)
        return
    head = bench_verify(args.config, args, steps=args.steps, warmup=args.warmup, headline=True)
    wl = head.pop("_wl")
    log(f"{head['workload']}: {head['ms_per_step']:.4f} ms/step ({head['launch']}), "
        f"step roofline {head['step_roofline']['frac']:.3f}")
    configs = {}
    for c in [int(c) for c in args.other_configs.split(",") if c.strip()]:
        if c == args.config:
            continue
        r = bench_verify(c, args, steps=max(args.steps, args.min_steps), warmup=max(args.warmup, 10))
        log(f"{r['workload']}: {r['ms_per_step']:.4f} ms/step ({r['launch']}), "
            f"step roofline {r['step_roofline']['frac']:.3f}")
        configs[r["workload"]] = r

    out = {
        "metric": "tree-verify nodes/sec + accepted tok/s at 1 GPU; % of HBM/MFMA roofline",
        "value": head["nodes_s"],
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic: seeded random-init weights N(0,0.02), KV prefix and node states N(0,1), uniform tokens",
        "config": {"workload": head["workload"], "batch": head["batch"], "tree_nodes": head["tree_nodes"],
                   "max_tree_nodes": head["max_tree_nodes"], "prefix": max(head["prefix"]), **head["shape"],
                   "step": "tree_build + tree_verify + accept_commit", "launch": head["launch"],
                   "weight_layout": layout_name(args)},
        "roofline": head["lm_head_roofline"],
        "step_roofline": head["step_roofline"],
        "step_ms": head["step_ms"],
        "eager_step_ms": head["eager_step_ms"],
        "accepted_tok_s": head["accepted_tok_s"],
        "accepted_per_step": head["accepted_per_step"],
        "accepted_tok_s_planted_depth3": head["accepted_tok_s_planted_depth3"],
        "stage_ms_per_step": head["stage_ms_per_step"],
        "configs": configs,
    }
    if not args.no_eagle_step and head["dtype"] == "bf16":
        torch.cuda.empty_cache()
        out["eagle_step"] = bench_eagle_step(args)
    if not args.no_decode and head["dtype"] == "bf16":
        torch.cuda.empty_cache()
        out["decode"] = bench_decode(args)
    if args.pmc_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        out["pmc_calibration_copy_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_nodes)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
