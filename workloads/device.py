"""Upload a seeded workload to device memory (torch tensors).  No arithmetic of the method."""
import numpy as np


def to_tensor(a, device="cuda"):
    """numpy -> torch on device; uint16 arrays are bf16 bit patterns and become torch.bfloat16."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def upload(wl, device="cuda"):
    """Device copies of every array of a workloads.Workload; returns a dict of tensors."""
    t = {}
    t["weights"] = {k: to_tensor(v, device) for k, v in wl.weights.items()}
    t["draft_weights"] = {k: to_tensor(v, device) for k, v in wl.draft_weights.items()}
    t["k_cache"] = to_tensor(wl.k_cache, device)
    t["v_cache"] = to_tensor(wl.v_cache, device)
    t["prefix_len"] = to_tensor(wl.prefix_len.astype(np.int32), device)
    if wl.x is not None:
        t["x"] = to_tensor(wl.x, device)
    if wl.tree_off is not None:
        t["tree_off"] = to_tensor(wl.tree_off.astype(np.int32), device)
        t["parent"] = to_tensor(np.concatenate([np.asarray(p, dtype=np.int32) for p in wl.parents]), device)
        t["tokens"] = to_tensor(wl.tokens.astype(np.int32), device)
    if wl.dk_cache is not None:
        t["dk_cache"] = to_tensor(wl.dk_cache, device)
        t["dv_cache"] = to_tensor(wl.dv_cache, device)
        t["root_feature"] = to_tensor(wl.root_feature, device)
        t["root_token"] = to_tensor(wl.root_token.astype(np.int32), device)
    return t
