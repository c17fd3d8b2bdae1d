"""Counter-seeded generators for router rows, router bias, experts and tokens.

Every draw is keyed by (seed, tag, indices...) through NumPy's SeedSequence
and PCG64, so any single expert or token can be regenerated on its own (the
oracle regenerates only the experts a token selects).

Recipe (the value distributions of the workloads):
  * router weights  Wr[e, h] = fp32(N(0, 1) / sqrt(H))            -> N(0, 1/H)
  * router bias     b[e] = fp32(-s * ln r_e), r a random permutation of
                    1..E (a log-Zipf(s) prior over experts); absent when the
                    workload is unbiased
  * expert codes    uniform random bytes: every 2/3/4-bit code is then
                    uniform and independent, whatever the bit layout
  * expert scales   d = fp16(|N(0, 0.02^2)|), round-to-nearest-even; for
                    MXFP4 the E8M0 byte 127 + floor(log2 |N(0, 0.02^2)|) - 2,
                    clipped to [1, 254] (so 6 x 2^(e-127), the largest
                    element magnitude, is 0.75 to 1.5 times the drawn value)
  * tokens          x = bf16(fp32(N(0, 1))), round-to-nearest-even

Canonical expert record (the storage layout the library's create call
consumes): gate [I rows][H/32 blocks], up [I][H/32], down [H][I/32]; each
block is its code bytes followed by the little-endian fp16 scale (MXFP4: the
E8M0 scale byte).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import FORMATS, BLOCK, MXFP4, canonical_block_bytes

TAG_ROUTER, TAG_BIAS, TAG_EXPERT, TAG_SHARED, TAG_TOKEN = 1, 2, 3, 4, 5


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_weights(seed: int, layer: int, hidden: int, n_experts: int) -> np.ndarray:
    g = _rng(seed, TAG_ROUTER, layer)
    w = g.standard_normal((n_experts, hidden)) / np.sqrt(hidden)
    return w.astype(np.float32)


def router_bias(seed: int, layer: int, n_experts: int, s: float = 1.1) -> np.ndarray:
    g = _rng(seed, TAG_BIAS, layer)
    ranks = g.permutation(n_experts) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def _blocks(g, n_blocks: int, fmt: int, d_sigma: float = 0.02) -> np.ndarray:
    cb = FORMATS[fmt][1]
    codes = g.integers(0, 256, size=(n_blocks, cb), dtype=np.uint8)
    out = np.empty((n_blocks, canonical_block_bytes(fmt)), dtype=np.uint8)
    out[:, :cb] = codes
    if fmt == MXFP4:
        a = np.abs(d_sigma * g.standard_normal(n_blocks))
        e = 127 + np.floor(np.log2(np.maximum(a, 1e-30))) - 2
        out[:, cb] = np.clip(e, 1, 254).astype(np.uint8)
    else:
        d = np.abs(d_sigma * g.standard_normal(n_blocks)).astype(np.float16)
        out[:, cb:] = d.astype("<f2").view(np.uint8).reshape(n_blocks, 2)
    return out


def _expert_blocks(hidden: int, inter: int) -> int:
    return 2 * inter * (hidden // BLOCK) + hidden * (inter // BLOCK)


def expert_canonical(seed: int, layer: int, expert: int, hidden: int, inter: int,
                     fmt: int, d_sigma: float = 0.02) -> np.ndarray:
    """One routed expert's canonical record as a flat uint8 array."""
    g = _rng(seed, TAG_EXPERT, layer, expert)
    return _blocks(g, _expert_blocks(hidden, inter), fmt, d_sigma).reshape(-1)


def shared_canonical(seed: int, layer: int, hidden: int, inter: int, fmt: int,
                     d_sigma: float = 0.02) -> np.ndarray:
    g = _rng(seed, TAG_SHARED, layer)
    return _blocks(g, _expert_blocks(hidden, inter), fmt, d_sigma).reshape(-1)


def layer_canonical(seed: int, layer: int, hidden: int, inter: int, n_experts: int,
                    fmt: int, d_sigma: float = 0.02) -> np.ndarray:
    """All routed experts of a layer, [E, record_bytes] uint8, expert-id order."""
    rec = _expert_blocks(hidden, inter) * canonical_block_bytes(fmt)
    out = np.empty((n_experts, rec), dtype=np.uint8)

    def fill(e):
        out[e] = expert_canonical(seed, layer, e, hidden, inter, fmt, d_sigma)

    # each expert has its own generator, so the draws are independent of the thread count
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n_experts)))
    return out


def token_candidates(seed: int, stream: int, index: int, hidden: int, attempt: int = 0) -> np.ndarray:
    """Candidate activation row for token `index` of a stream: bf16 bits [H]."""
    g = _rng(seed, TAG_TOKEN, stream, index, attempt)
    return f32_to_bf16_bits(g.standard_normal(hidden).astype(np.float32))
