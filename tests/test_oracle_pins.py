"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed independently of its own
code: hand-derived block patterns, an independent packer, a scalar dense
reference written from the definitions, closed forms, exact scaling
invariants and the defining properties of top-k and the stable sort.
"""

import json
import os
import struct

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle as O
from moe_synth import generate as G

HERE = os.path.dirname(os.path.abspath(__file__))
OFFSETS = {2: 1.5, 3: 3.5, 4: 8.0}        # w = d * (q - c), from the format definitions
CODE_BYTES = {2: 8, 3: 12, 4: 16, 5: 16}
BITS = {2: 2, 3: 3, 4: 4, 5: 4}
SCALE_BYTES = {2: 2, 3: 2, 4: 2, 5: 1}
MXFP4 = 5

# FP4 E2M1 element values of codes 0..15 as tabulated in the OCP Microscaling
# Formats (MX) v1.0 specification (section 5.3.3): 0, 0.5, 1, 1.5, 2, 3, 4, 6,
# then the same with the sign bit set
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


# ------------------------------------------------------------------ O1 unpack
def test_block_patterns_golden():
    cases = json.load(open(os.path.join(HERE, "golden", "block_patterns.json")))["cases"]
    for c in cases:
        blk = np.frombuffer(bytes.fromhex(c["codes_hex"]) + bytes.fromhex(c["d_fp16_hex"])[::-1],
                            dtype=np.uint8)
        w = O.dequant_blocks(blk[None, :], c["fmt"])      # one block -> 32 weights
        np.testing.assert_array_equal(w, np.array(c["w"], dtype=np.float64), err_msg=c["name"])


def _pack_codes(codes, bits):
    """Independent scalar packer: code j at bits [bits*j, bits*j+bits)."""
    v = 0
    for j, q in enumerate(codes):
        v |= int(q) << (bits * j)
    return v.to_bytes(len(codes) * bits // 8, "little")


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_pack_unpack_roundtrip(fmt):
    rng = np.random.default_rng(7 + fmt)
    codes = rng.integers(0, 1 << BITS[fmt], size=(50, 32))
    packed = np.stack([np.frombuffer(_pack_codes(c, BITS[fmt]), dtype=np.uint8) for c in codes])
    assert packed.shape == (50, CODE_BYTES[fmt])
    np.testing.assert_array_equal(O.unpack_codes(packed, BITS[fmt]), codes)


# ------------------------------------------------------------------ MXFP4 (OCP MX v1.0)
def _torch_fp4_reference():
    """PyTorch's own FP4 unpacking reference (its testing helpers import
    expecttest only for test-case classes; a stand-in module is enough)."""
    import sys
    import types
    if "expecttest" not in sys.modules:
        stub = types.ModuleType("expecttest")
        stub.TestCase = object
        sys.modules["expecttest"] = stub
    from torch.testing._internal.common_quantized import _floatx_unpacked_to_f32
    return _floatx_unpacked_to_f32


def test_e2m1_matches_pytorch_reference():
    torch = pytest.importorskip("torch")
    try:
        ref_fn = _torch_fp4_reference()
    except Exception as e:                      # pragma: no cover - depends on the torch build
        pytest.skip(f"PyTorch FP4 reference unavailable: {e}")
    ref = ref_fn(torch.arange(16, dtype=torch.uint8), 2, 1).double().numpy()
    got = O.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def test_e2m1_matches_the_spec_table():
    got = O.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(got, np.array(E2M1_SPEC))
    np.testing.assert_array_equal(np.signbit(got), np.signbit(np.array(E2M1_SPEC)))


def test_e8m0_matches_pytorch_float8_e8m0fnu():
    torch = pytest.importorskip("torch")
    e = np.arange(255, dtype=np.uint8)             # 255 is NaN in both
    ref = torch.from_numpy(e).view(torch.float8_e8m0fnu).float().double().numpy()
    np.testing.assert_array_equal(O.e8m0_value(e), ref)
    assert np.isnan(O.e8m0_value(255))


def test_mxfp4_block_golden():
    # hand-built blocks: codes 0..15 twice; scale bytes 127 (x1), 130 (x8), 120 (x2^-7)
    codes = bytes((2 * j) | ((2 * j + 1) << 4) for j in range(8)) * 2
    for e, scale in [(127, 1.0), (130, 8.0), (120, 2.0 ** -7)]:
        blk = np.frombuffer(codes + bytes([e]), dtype=np.uint8)
        w = O.dequant_blocks(blk[None, :], MXFP4)
        np.testing.assert_array_equal(w, scale * np.array(E2M1_SPEC * 2))


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_levels_are_the_stated_grid(fmt):
    # every reachable weight is d*(q-c) for an integer code 0 <= q < 2^b
    # (MXFP4: 2^(e-127) times an E2M1 value)
    rng = np.random.default_rng(fmt)
    blocks = rng.integers(0, 256, size=(400, CODE_BYTES[fmt] + SCALE_BYTES[fmt]), dtype=np.uint8)
    if fmt == MXFP4:
        blocks[:, -1] = 127
    else:
        blocks[:, -2:] = np.frombuffer(np.float16(1.0).tobytes(), dtype=np.uint8)
    w = O.dequant_blocks(blocks, fmt)
    levels = np.unique(w)
    want = np.unique(np.array(E2M1_SPEC)) if fmt == MXFP4 else np.arange(1 << fmt) - OFFSETS[fmt]
    np.testing.assert_array_equal(levels, want)


# ------------------------------------------------------------------ dense scalar reference
def _scalar_matrix(blocks, fmt):
    """Scalar, per-weight expansion of a [rows][nblk][Bq] block array."""
    cb, bits = CODE_BYTES[fmt], BITS[fmt]
    rows, nblk, _ = blocks.shape
    out = np.zeros((rows, nblk * 32))
    for r in range(rows):
        for b in range(nblk):
            raw = bytes(blocks[r, b])
            bitval = int.from_bytes(raw[:cb], "little")
            for j in range(32):
                q = (bitval >> (bits * j)) & ((1 << bits) - 1)
                if fmt == MXFP4:
                    out[r, b * 32 + j] = 2.0 ** (raw[cb] - 127) * E2M1_SPEC[q]
                else:
                    (d,) = struct.unpack("<e", raw[cb:cb + 2])
                    out[r, b * 32 + j] = d * (q - OFFSETS[fmt])
    return out


def _dense_reference(x, wr, b, records, shared, H, I, k, fmt, residual):
    """Every expert on every token, then masked by the top-k set."""
    T, E = x.shape[0], wr.shape[0]
    bq = CODE_BYTES[fmt] + SCALE_BYTES[fmt]
    n_gu = I * (H // 32) * bq

    def expand(rec):
        rec = np.asarray(rec)
        g = _scalar_matrix(rec[:n_gu].reshape(I, H // 32, bq), fmt)
        u = _scalar_matrix(rec[n_gu:2 * n_gu].reshape(I, H // 32, bq), fmt)
        d = _scalar_matrix(rec[2 * n_gu:].reshape(H, I // 32, bq), fmt)
        return g, u, d

    def ffn(xt, g, u, d):
        gv = [sum(g[i, h] * xt[h] for h in range(H)) for i in range(I)]
        uv = [sum(u[i, h] * xt[h] for h in range(H)) for i in range(I)]
        a = [gv[i] / (1.0 + np.exp(-gv[i])) * uv[i] for i in range(I)]
        return np.array([sum(d[h, i] * a[i] for i in range(I)) for h in range(H)])

    mats = [expand(r) for r in records]
    out = np.zeros((T, H))
    for t in range(T):
        logit = [sum(float(x[t, h]) * float(wr[e, h]) for h in range(H)) + (0.0 if b is None else float(b[e]))
                 for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-logit[e], e))[:k]
        m = max(logit[e] for e in chosen)
        z = {e: np.exp(logit[e] - m) for e in chosen}
        s = sum(z.values())
        for e in range(E):               # all experts evaluated, masked afterwards
            y = ffn(x[t], *mats[e])
            if e in z:
                out[t] += (z[e] / s) * y
        if shared is not None:
            out[t] += ffn(x[t], *expand(shared))
        if residual:
            out[t] += x[t]
    return out


@pytest.mark.parametrize("fmt,biased,shared,residual", [
    (2, False, False, False), (2, True, False, True), (3, True, False, False), (4, True, True, False),
    (5, True, True, True)])
def test_oracle_matches_scalar_dense_reference(fmt, biased, shared, residual):
    H, I, E, k, T = 64, 32, 5, 2, 3
    wr = G.router_weights(11, 0, H, E)
    b = G.router_bias(11, 0, E) if biased else None
    recs = [G.expert_canonical(11, 0, e, H, I, fmt) for e in range(E)]
    sh = G.shared_canonical(11, 0, H, I, fmt) if shared else None
    x = G.bf16_bits_to_f32(np.stack([G.token_candidates(11, 0, t, H) for t in range(T)])).astype(np.float64)
    got, _ = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, k, fmt, shared_record=sh, residual=residual)
    ref = _dense_reference(x, wr, b, recs, sh, H, I, k, fmt, residual)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


# ------------------------------------------------------------------ O2-O4 routing
def test_topk_defining_property_and_order():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 37))
    l[5, :] = 0.0                                   # all ties -> lowest ids
    for k in (1, 4, 37):
        idx, gap = O.select_topk(l, k)
        assert idx.shape == (200, k)
        assert np.all(np.diff(idx, axis=1) > 0)     # ascending, distinct
        for t in range(200):
            sel = l[t, idx[t]]
            rest = np.delete(l[t], idx[t])
            if rest.size:
                assert sel.min() >= rest.max()
                assert gap[t] == pytest.approx(sel.min() - rest.max())
        np.testing.assert_array_equal(idx[5], np.arange(k))


def test_weights_sum_to_one_and_follow_logits():
    rng = np.random.default_rng(4)
    l = 3.0 * rng.standard_normal((100, 64))
    idx, _ = O.select_topk(l, 10)
    w = O.routing_weights(l, idx)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    sel = np.take_along_axis(l, idx, axis=1)
    # the ratio of two weights is exp of the logit difference
    np.testing.assert_allclose(w[:, 0] / w[:, 1], np.exp(sel[:, 0] - sel[:, 1]), rtol=1e-12)


def test_bias_enters_selection():
    H, E = 32, 8
    x = np.zeros((1, H))
    wr = np.zeros((E, H), dtype=np.float32)
    b = np.array([0, 5, 0, 7, 0, 0, 6, 0], dtype=np.float32)
    _, idx, w, _ = O.route(x, wr, b, 3)
    np.testing.assert_array_equal(idx[0], [1, 3, 6])
    e = np.exp([5.0 - 7.0, 0.0, 6.0 - 7.0])
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-15)


# ------------------------------------------------------------------ special cases
def _tiny_layer(fmt, E=6, H=64, I=32, T=4, seed=21):
    wr = G.router_weights(seed, 0, H, E)
    b = G.router_bias(seed, 0, E)
    recs = [G.expert_canonical(seed, 0, e, H, I, fmt) for e in range(E)]
    x = G.bf16_bits_to_f32(np.stack([G.token_candidates(seed, 0, t, H) for t in range(T)])).astype(np.float64)
    return wr, b, recs, x


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_k_equals_E_is_the_dense_softmax_mixture(fmt):
    H, I, E = 64, 32, 6
    wr, b, recs, x = _tiny_layer(fmt, E, H, I)
    got, _ = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, E, fmt)
    p = scipy_softmax(x @ wr.T.astype(np.float64) + b.astype(np.float64), axis=1)
    ys = [O.expert_ffn(x, *O.dequant_expert(recs[e], H, I, fmt)) for e in range(E)]
    ref = sum(p[:, e:e + 1] * ys[e] for e in range(E))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_k1_is_the_argmax_expert_exactly(fmt):
    H, I, E = 64, 32, 6
    wr, b, recs, x = _tiny_layer(fmt, E, H, I)
    got, info = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, 1, fmt)
    assert np.all(info["w"] == 1.0)
    best = np.argmax(x @ wr.T.astype(np.float64) + b.astype(np.float64), axis=1)
    for t in range(x.shape[0]):
        y = O.expert_ffn(x[t:t + 1], *O.dequant_expert(recs[best[t]], H, I, fmt))
        # weight exactly 1; BLAS may round a 1-row product differently
        np.testing.assert_allclose(got[t], y[0], rtol=1e-13, atol=1e-18)


def _scale_matrix(rec, H, I, fmt, which, factor_bits):
    """Return a copy of rec with every fp16 scale of one matrix replaced via fn."""
    bq = CODE_BYTES[fmt] + 2
    rec = np.array(rec, copy=True)
    n_gu = I * (H // 32) * bq
    lo, hi = {"gate": (0, n_gu), "up": (n_gu, 2 * n_gu), "down": (2 * n_gu, rec.size)}[which]
    blocks = rec[lo:hi].reshape(-1, bq)
    d = np.ascontiguousarray(blocks[:, -2:]).view("<f2")[:, 0]
    blocks[:, -2:] = factor_bits(d).astype("<f2").view(np.uint8).reshape(-1, 2)
    rec[lo:hi] = blocks.reshape(-1)
    return rec


@pytest.mark.parametrize("which", ["up", "down"])
def test_doubling_up_or_down_scales_doubles_output_exactly(which):
    H, I, E, k, fmt = 64, 32, 6, 2, 3
    wr, b, recs, x = _tiny_layer(fmt, E, H, I)
    base, _ = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, k, fmt)
    rec2 = [_scale_matrix(r, H, I, fmt, which, lambda d: d * np.float16(2)) for r in recs]
    got, _ = O.moe_layer(x, wr, b, lambda e: rec2[e], H, I, k, fmt)
    np.testing.assert_array_equal(got, 2.0 * base)


def test_zero_gate_scales_give_zero_output():
    H, I, E, k, fmt = 64, 32, 6, 2, 2
    wr, b, recs, x = _tiny_layer(fmt, E, H, I)
    rec0 = [_scale_matrix(r, H, I, fmt, "gate", lambda d: d * np.float16(0)) for r in recs]
    got, _ = O.moe_layer(x, wr, b, lambda e: rec0[e], H, I, k, fmt)
    assert np.all(got == 0.0)


def test_relabelling_experts_leaves_output_unchanged():
    H, I, E, k, fmt = 64, 32, 6, 3, 4
    wr, b, recs, x = _tiny_layer(fmt, E, H, I)
    base, info = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, k, fmt)
    pi = np.array([3, 0, 5, 1, 4, 2])
    got, info2 = O.moe_layer(x, wr[pi], b[pi], lambda e: recs[pi[e]], H, I, k, fmt)
    np.testing.assert_allclose(got, base, rtol=1e-13, atol=1e-16)
    np.testing.assert_array_equal(np.sort(pi[info2["idx"]], axis=1), info["idx"])


def test_constant_expert_closed_form():
    # One expert, k = 1, Q4, d = 1: gate codes 9 (w = 1), up codes 10 (w = 2),
    # down codes 7 (w = -1).  With S = sum_h x_h: g_i = S, u_i = 2S,
    # a_i = silu(S) * 2S and y_h = -I * silu(S) * 2S for every h.
    H, I, fmt = 64, 32, 4
    one = np.frombuffer(np.float16(1.0).tobytes(), dtype=np.uint8)

    def mat(rows, cols, code):
        blk = np.concatenate([np.full(16, code | (code << 4), dtype=np.uint8), one])
        return np.tile(blk, rows * (cols // 32))

    rec = np.concatenate([mat(I, H, 9), mat(I, H, 10), mat(H, I, 7)])
    x = (np.linspace(-0.5, 0.5, H) - 1.0 / H)[None, :]     # S = -1: silu far from linear
    out, _ = O.moe_layer(x, np.zeros((1, H), np.float32), None, lambda e: rec, H, I, 1, fmt)
    S = x.sum()
    expect = -I * (S / (1.0 + np.exp(-S))) * 2.0 * S
    np.testing.assert_allclose(out[0], np.full(H, expect), rtol=1e-13)
    # swapping the roles of gate and up would give -I * silu(2S) * S instead
    assert abs(expect - (-I * (2 * S / (1 + np.exp(-2 * S))) * S)) > 1e-3


# ------------------------------------------------------------------ O7 permute
def test_permute_invariants_and_roundtrip():
    rng = np.random.default_rng(9)
    T, E, k = 300, 40, 5
    idx = np.sort(np.stack([rng.choice(E, size=k, replace=False, p=np.arange(1, E + 1) / (E * (E + 1) / 2))
                            for _ in range(T)]), axis=1)
    counts, offsets, perm, inv = O.permute(idx, E)
    P = T * k
    assert counts.sum() == P and offsets[0] == 0 and offsets[-1] == P
    assert np.all(np.diff(offsets) == counts)
    np.testing.assert_array_equal(np.sort(perm), np.arange(P))
    np.testing.assert_array_equal(perm[inv], np.arange(P))
    flat = idx.reshape(-1)
    keys = list(zip(flat[perm], perm))
    assert keys == sorted(keys)                              # stable by (expert, p)
    for e in range(E):
        assert np.all(flat[perm[offsets[e]:offsets[e + 1]]] == e)
    # unpermute(permute(X)) with unit weights sums k copies of each row
    X = rng.standard_normal((T, 6))
    Xs = X[perm // k]                                        # rows in slot order
    back = np.zeros_like(X)
    for p in range(P):
        back[p // k] += Xs[inv[p]]
    np.testing.assert_array_equal(back, k * X)


def test_stack_applies_residual_per_layer():
    H, I, E, k, fmt = 64, 32, 6, 2, 3
    layers = []
    for l in range(3):
        wr = G.router_weights(5, l, H, E)
        b = G.router_bias(5, l, E)
        recs = [G.expert_canonical(5, l, e, H, I, fmt) for e in range(E)]
        layers.append((wr, b, (lambda rs: (lambda e: rs[e]))(recs)))
    x0 = G.bf16_bits_to_f32(G.token_candidates(5, 0, 0, H)).astype(np.float64)[None, :]
    h, infos = O.moe_stack(x0, layers, H, I, k, fmt)
    ref = x0.copy()
    for wr, b, rec in layers:
        y, _ = O.moe_layer(ref, wr, b, rec, H, I, k, fmt)
        ref = ref + y
    np.testing.assert_array_equal(h, ref)
    assert len(infos) == 3
