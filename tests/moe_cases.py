"""Shared helpers of the GPU parity tests: seeded layers and tokens, the
oracle reference on the same inputs, and the HIP layer through the C ABI."""

import numpy as np
import torch

import oracle as O
from moe_synth import generate as G

DECODE_TOL = 1e-5      # rel-L2, fp32 decode path vs fp64 oracle
PREFILL_TOL = 2e-2     # rel-L2, 16-bit-MFMA prefill path vs fp64 oracle
MIN_GAP = 1e-2         # logit gap at rank k required of every generated token


class HostLayer:
    """One layer's seeded inputs on the host (canonical records, router)."""

    def __init__(self, seed, layer, H, I, E, k, fmt, biased, n_shared=0, materialise=True):
        self.seed, self.layer = seed, layer
        self.H, self.I, self.E, self.k, self.fmt, self.n_shared = H, I, E, k, fmt, n_shared
        self.wr = G.router_weights(seed, layer, H, E)
        self.b = G.router_bias(seed, layer, E) if biased else None
        self.canon = G.layer_canonical(seed, layer, H, I, E, fmt) if materialise else None
        self.shared = G.shared_canonical(seed, layer, H, I, fmt) if n_shared else None

    def record(self, e):
        if self.canon is not None:
            return self.canon[e]
        return G.expert_canonical(self.seed, self.layer, e, self.H, self.I, self.fmt)

    def oracle(self, x, residual=False):
        return O.moe_layer(np.asarray(x, np.float64), self.wr, self.b, self.record, self.H, self.I,
                           self.k, self.fmt, shared_record=self.shared, residual=residual)

    def logits(self, x):
        return O.router_logits(np.asarray(x, np.float64), self.wr, self.b)

    def mixture(self, x, idx, w):
        """The layer's output for given ids and routing weights (the oracle's
        expert FFNs, weighted as the layer defines), e.g. the weights a device
        router computed: separates the expert path's precision from the
        router's rounding."""
        x = np.asarray(x, np.float64)
        out = np.zeros((x.shape[0], self.H), dtype=np.float64)
        for e in np.unique(idx):
            rows, cols = np.nonzero(idx == e)
            wg, wu, wd = O.dequant_expert(self.record(int(e)), self.H, self.I, self.fmt)
            out[rows] += np.asarray(w, np.float64)[rows, cols][:, None] * O.expert_ffn(x[rows], wg, wu, wd)
        if self.shared is not None:
            wg, wu, wd = O.dequant_expert(self.shared, self.H, self.I, self.fmt)
            out += O.expert_ffn(x, wg, wu, wd)
        return out


def tokens(hl, stream, T, min_gap=MIN_GAP, max_attempts=200):
    """Gap-filtered bf16 tokens for layer hl: returns (bits uint16 [T,H], fp64 values)."""
    H = hl.H
    x = np.stack([G.token_candidates(hl.seed, stream, t, H, 0) for t in range(T)])
    attempt = np.zeros(T, dtype=np.int64)
    for _ in range(max_attempts):
        xf = G.bf16_bits_to_f32(x).astype(np.float64)
        _, gap = O.select_topk(hl.logits(xf), hl.k)
        bad = np.nonzero(gap < min_gap)[0]
        if bad.size == 0:
            return x, xf
        for t in bad:
            attempt[t] += 1
            x[t] = G.token_candidates(hl.seed, stream, int(t), H, int(attempt[t]))
    raise RuntimeError("could not draw tokens with the required logit gap")


def to_device_bf16(bits, dev):
    return torch.from_numpy(bits.astype(np.int16)).to(dev).view(torch.bfloat16)


def device_layer(hl, max_tokens, dev):
    from quantized_moe_expert_gemv_amd import binding as B
    cfg = B.make_config(hl.H, hl.I, hl.E, hl.k, hl.n_shared, hl.fmt, max_tokens)
    wr = torch.from_numpy(hl.wr).to(dev)
    b = None if hl.b is None else torch.from_numpy(hl.b).to(dev)
    canon = torch.from_numpy(np.ascontiguousarray(hl.canon).reshape(-1)).to(dev)
    sh = None if hl.shared is None else torch.from_numpy(hl.shared).to(dev)
    layer = B.StrataMoE(cfg, wr, b, canon, sh)
    del canon, sh
    return layer


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def row_rel_l2(got, ref):
    """Relative L2 error of every token row: ||got_t - ref_t|| / ||ref_t||."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)


def check_rows(got, ref, tol, what=""):
    """The call's rel-L2 over all compared rows and the worst single row, both
    within tol (a token with a wrong row cannot hide in the pooled norm).
    Returns (pooled, worst row)."""
    pooled = rel_l2(got, ref)
    rows = row_rel_l2(got, ref)
    worst = float(rows.max())
    print(f"{what} rows {rows.size}: rel-L2 {pooled:.3e}, worst row {worst:.3e} "
          f"(token {int(rows.argmax())}), bound {tol:g}", flush=True)
    assert np.isfinite(pooled) and pooled <= tol, (what, pooled)
    assert np.isfinite(worst) and worst <= tol, (what, worst, int(rows.argmax()))
    return pooled, worst


def tile_tokens(idx, n_experts, n_shared=0, rows=128, seed=0):
    """Tokens that put at least one row into every 128-slot GEMM tile.

    The expert GEMMs of the grouped path work on tiles of `rows` consecutive
    slots of one expert in the stable (expert, pair) order (the permutation
    of the routing), full tiles first and then the expert's remainder; the
    shared expert's slots follow, one per token.  For every such tile this
    picks a random slot and the last slot, and returns the sorted tokens that
    own them."""
    rng = np.random.default_rng(seed)
    idx = np.asarray(idx)
    T, k = idx.shape
    counts, offsets, perm, _ = O.permute(idx, n_experts)
    toks = set()
    for e in range(n_experts):
        c = int(counts[e])
        for j0 in range(0, c, rows):
            n = min(rows, c - j0)
            for slot in (offsets[e] + j0 + int(rng.integers(n)), offsets[e] + j0 + n - 1):
                toks.add(int(perm[slot]) // k)
    if n_shared:
        for j0 in range(0, T, rows):
            n = min(rows, T - j0)
            toks.add(j0 + int(rng.integers(n)))
            toks.add(j0 + n - 1)
    return np.array(sorted(toks), dtype=np.int64)


def check_route(layer, hl, x_dev, x_f64, flags=0, w_atol=2e-6):
    """Route outputs vs the oracle: ids, permutation and offsets bit-exact."""
    idx, w, perm, offs = layer.route(x_dev, flags=flags)
    torch.cuda.synchronize()
    _, oidx, ow, _ = O.route(x_f64, hl.wr, hl.b, hl.k)
    counts, ooffs, operm, _ = O.permute(oidx, hl.E)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    np.testing.assert_array_equal(perm.cpu().numpy(), operm)
    np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=0, atol=w_atol)
    return oidx
