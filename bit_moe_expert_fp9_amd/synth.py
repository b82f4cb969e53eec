"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no fp9 rounding, no decode, no GEMV).  Both the library
path and the oracle take its float32 arrays and quantize them on their own.

Recipe (the pages measure on trained DeepSeek-V3.2 weights and their own
prompts, neither available; these draws stand in, with the layer's shapes):
  * weights: N(0, 0.02) float32, one independent stream per
    (seed, workload, layer, expert, matrix), matrix 0 = gate, 1 = up, 2 = down;
  * activations: N(0, 1) float32 per (seed, workload, layer, step);
  * routing per token: 8 (top_k) distinct ids drawn uniformly from the routed
    experts, weights = softmax of top_k N(0, 1) draws, per
    (seed, workload, layer, step).
Every stream is numpy's PCG64 seeded by SeedSequence of the tuple above.

For layers too large to draw on the host in reasonable time (the 16-layer
stack holds 4112 experts), weights_device draws the same N(0, 0.02)
distribution on the GPU with torch's Philox generator, seeded from the same
key.  It is a different stream from `weights` (the values differ); the oracle
side takes those device-drawn float32 values, copied to the host, and
quantizes them itself.
"""

import numpy as np

WEIGHT_STD = 0.02
GATE, UP, DOWN = 0, 1, 2


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def weights(seed, workload, layer, expert, matrix, shape, out=None):
    """N(0, 0.02) float32 of the given shape (optionally written into `out`)."""
    rng = _rng(seed, workload, layer, expert, matrix, 0)
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    out *= np.float32(WEIGHT_STD)
    return out


def device_seed(*key):
    """63-bit torch generator seed derived from a key tuple."""
    state = np.random.SeedSequence([int(k) for k in key]).generate_state(2, np.uint32)
    return (int(state[0]) | (int(state[1]) << 32)) & ((1 << 63) - 1)


def weights_device(seed, workload, layer, expert, matrix, shape, device="cuda"):
    """N(0, 0.02) float32 of the given shape drawn on `device` (torch Philox)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(seed, workload, layer, expert, matrix, 3))
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out.mul_(WEIGHT_STD)
    return out


def fp8_weights(seed, workload, layer, expert, matrix, shape, block=128):
    """Synthetic fp8 checkpoint matrix: (codes uint8 [rows, cols], scales float32
    [ceil(rows/block), ceil(cols/block)]).  Codes are uniform over the 254
    non-NaN E4M3 codes (every exponent, both signs); scales are 10^U(-5, -3)
    per block.  Bytes and scales are drawn, nothing is rounded here."""
    rng = _rng(seed, workload, layer, expert, matrix, 4)
    rows, cols = shape
    codes = rng.integers(0, 254, size=shape, dtype=np.int64)
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)  # skip 0x7F and 0xFF
    nb = (-(-rows // block), -(-cols // block))
    scales = (10.0 ** rng.uniform(-5.0, -3.0, size=nb)).astype(np.float32)
    return codes, scales


def activations(seed, workload, layer, step, T, hidden):
    """x [T, hidden] ~ N(0, 1), float32."""
    rng = _rng(seed, workload, layer, step, 1)
    return rng.standard_normal((T, hidden), dtype=np.float32)


def routing(seed, workload, layer, step, T, n_routed, top_k):
    """(ids int32 [T, top_k], w float32 [T, top_k]) for one decode step."""
    rng = _rng(seed, workload, layer, step, 2)
    ids = np.stack([rng.choice(n_routed, size=top_k, replace=False) for _ in range(T)])
    z = rng.standard_normal((T, top_k))
    w = np.exp(z - z.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def expert_shapes(hidden, inter):
    """(gate, up, down) matrix shapes of one expert."""
    return (inter, hidden), (inter, hidden), (hidden, inter)
