"""Seeded synthetic inputs for the MoE layer (tests and benchmark).

This module only draws random numbers; it holds none of the layer's
arithmetic.  Both the oracle-side tests and the HIP-side tests take their
inputs from here, so the two sides see identical bytes.

Recipe (shapes follow the K3 layer: hidden 7168, 896 routed experts of
intermediate 1536, top-16, 2 shared experts):
  * every tensor comes from numpy PCG64 seeded with [seed, layer, tensor, index]
    so any single expert can be regenerated on its own;
  * MXFP4 code bytes are uniform over 0..255 (both nibbles uniform over the
    16 E2M1 codes), E8M0 scale bytes uniform over 118..126;
  * bf16 tensors are float32 normal draws rounded to nearest-even bf16:
    router N(0, 0.02), shared experts N(0, 0.02), activations N(0, 1),
    RMSNorm gain 1 + N(0, 0.01); the router bias is float32 N(0, 0.5).
"""

import numpy as np

T_X, T_ROUTER, T_EXPERT, T_SHARED, T_BIAS, T_GAMMA = range(6)

K3 = dict(hidden=7168, inter=1536, n_experts=896, top_k=16, n_shared=2)
TINY = dict(hidden=256, inter=64, n_experts=32, top_k=4, n_shared=1)


def rng(seed, layer, tensor, index=0):
    return np.random.default_rng([int(seed), int(layer), int(tensor), int(index)])


def to_bf16_bits(a32):
    """float32 -> bf16 bit patterns, nearest-even (finite inputs)."""
    b = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def normal_bf16(g, shape, std, mean=0.0):
    a = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if mean:
        a = a + np.float32(mean)
    return to_bf16_bits(a)


def record_bytes(hidden, inter):
    return 3 * (hidden * inter // 2 + hidden * inter // 32)


def expert_record(seed, layer, e, hidden, inter, out=None):
    """Bytes of expert e: six tensors (gate, up, down) x (codes, scales)."""
    n_codes = hidden * inter // 2
    n_scales = hidden * inter // 32
    nbytes = 3 * (n_codes + n_scales)
    if out is None:
        out = np.empty(nbytes, dtype=np.uint8)
    g = rng(seed, layer, T_EXPERT, e)
    off = 0
    for _ in range(3):
        raw = g.integers(0, 2 ** 64, size=(n_codes + 7) // 8, dtype=np.uint64)
        out[off:off + n_codes] = raw.view(np.uint8)[:n_codes]
        off += n_codes
        out[off:off + n_scales] = g.integers(118, 127, size=n_scales, dtype=np.uint8)
        off += n_scales
    return out


def router_weight(seed, layer, n_experts, hidden, std=0.02):
    return normal_bf16(rng(seed, layer, T_ROUTER), (n_experts, hidden), std)


def router_bias(seed, layer, n_experts, std=0.5):
    return rng(seed, layer, T_BIAS).standard_normal(n_experts, dtype=np.float32) * np.float32(std)


def shared_expert(seed, layer, s, hidden, inter, std=0.02):
    g = rng(seed, layer, T_SHARED, s)
    return (normal_bf16(g, (inter, hidden), std),
            normal_bf16(g, (inter, hidden), std),
            normal_bf16(g, (hidden, inter), std))


def activations(seed, n_tokens, hidden):
    """bf16 N(0,1) token rows; the i-th timed input uses seed 1000 + i."""
    return normal_bf16(rng(seed, 0, T_X), (n_tokens, hidden), 1.0)


def rms_gamma(seed, layer, hidden):
    return normal_bf16(rng(seed, layer, T_GAMMA), (hidden,), 0.01, mean=1.0)
