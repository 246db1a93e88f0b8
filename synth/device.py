"""Upload seeded synthetic layers to device memory (torch tensors).

Pure plumbing around synth's generators: bytes are generated on the host
(threads, one expert at a time) and copied to device buffers owned by torch.
"""

import concurrent.futures as cf

import numpy as np
import torch

from . import (activations, expert_record, record_bytes, rms_gamma, router_bias, router_weight,
               shared_expert)


def _u16(a, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def upload_experts(seed, layer, n_experts, hidden, inter, device, chunk=32, threads=8):
    """uint8 device tensor [E, record_bytes] of all expert records."""
    rb = record_bytes(hidden, inter)
    out = torch.empty((n_experts, rb), dtype=torch.uint8, device=device)
    pinned = [torch.empty((chunk, rb), dtype=torch.uint8).pin_memory() for _ in range(2)]
    events = [None, None]
    with cf.ThreadPoolExecutor(threads) as ex:
        for i, e0 in enumerate(range(0, n_experts, chunk)):
            buf = pinned[i % 2]
            if events[i % 2] is not None:
                events[i % 2].synchronize()
            n = min(chunk, n_experts - e0)
            host = buf.numpy()
            list(ex.map(lambda j: expert_record(seed, layer, e0 + j, hidden, inter, out=host[j]),
                        range(n)))
            out[e0:e0 + n].copy_(buf[:n], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            events[i % 2] = ev
    torch.cuda.synchronize()
    return out


def upload_layer(cfg, seed=0, layer=0, device="cuda", bias=False, n_experts_resident=None):
    """Device tensors of one synthetic layer.

    cfg: dict(hidden, inter, n_experts, top_k, n_shared).  Returns a dict of
    torch tensors (router_w int16 [E,H], experts uint8 [E,rec], shared_* int16,
    router_bias fp32 or None) plus the host copies the oracle needs (router_w
    and shared as uint16 numpy, bias float32 numpy).
    """
    H, I, E, S = cfg["hidden"], cfg["inter"], cfg["n_experts"], cfg["n_shared"]
    wr = router_weight(seed, layer, E, H)
    shared = [shared_expert(seed, layer, s, H, I) for s in range(S)]
    b = router_bias(seed, layer, E) if bias else None
    d = {
        "host_router_w": wr,
        "host_shared": shared,
        "host_bias": b,
        "router_w": _u16(wr, device),
        "experts": upload_experts(seed, layer, E, H, I, device),
        "router_bias": None if b is None else torch.from_numpy(b).to(device),
        "shared_gate": None, "shared_up": None, "shared_down": None,
    }
    if S:
        d["shared_gate"] = _u16(np.stack([s[0] for s in shared]), device)
        d["shared_up"] = _u16(np.stack([s[1] for s in shared]), device)
        d["shared_down"] = _u16(np.stack([s[2] for s in shared]), device)
    return d


def upload_tokens(seed, n_tokens, hidden, device="cuda"):
    x = activations(seed, n_tokens, hidden)
    return x, _u16(x, device)


def upload_gamma(seed, layer, hidden, device="cuda"):
    g = rms_gamma(seed, layer, hidden)
    return g, _u16(g, device)
