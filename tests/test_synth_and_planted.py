"""Generator determinism / distribution checks, and planted-mistake checks.

The planted-mistake tests swap a plausible bug into the oracle (on the CPU,
through monkeypatch) and assert that at least one independent pin rejects
it, so the pins are shown to be sharp enough.
"""

import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as OM
from moe_synth import generate as G, WORKLOADS
from tests.test_oracle_pins import _dense_reference


def test_generators_are_deterministic_and_keyed():
    a = G.expert_canonical(3, 1, 7, 256, 256, 3)
    b = G.expert_canonical(3, 1, 7, 256, 256, 3)
    c = G.expert_canonical(3, 1, 8, 256, 256, 3)
    assert a.dtype == np.uint8 and np.array_equal(a, b) and not np.array_equal(a, c)
    np.testing.assert_array_equal(G.token_candidates(1, 2, 3, 64), G.token_candidates(1, 2, 3, 64))
    assert not np.array_equal(G.token_candidates(1, 2, 3, 64), G.token_candidates(1, 2, 3, 64, attempt=1))
    np.testing.assert_array_equal(G.router_bias(4, 0, 16), G.router_bias(4, 0, 16))


def test_value_distributions():
    wr = G.router_weights(0, 0, 2560, 512)
    assert wr.dtype == np.float32 and abs(wr.var() * 2560 - 1) < 0.01
    b = G.router_bias(0, 0, 512)
    np.testing.assert_allclose(np.sort(b)[::-1], -1.1 * np.log(np.arange(1, 513)), rtol=1e-6)
    rec = G.expert_canonical(0, 0, 0, 2560, 512, 2).reshape(-1, 10)
    d = np.ascontiguousarray(rec[:, 8:]).view("<f2")[:, 0].astype(np.float64)
    assert np.all(d >= 0) and abs(np.sqrt((d ** 2).mean()) - 0.02) < 5e-4
    assert abs(rec[:, :8].mean() - 127.5) < 0.5
    x = G.bf16_bits_to_f32(G.token_candidates(0, 0, 0, 4096))
    assert abs(x.std() - 1) < 0.05
    # MXFP4: 16 code bytes then one E8M0 byte 127 + floor(log2 |N(0, 0.02^2)|) - 2
    mx = G.expert_canonical(0, 0, 0, 2560, 512, 5).reshape(-1, 17)
    e = mx[:, 16].astype(np.int64)
    assert e.min() >= 1 and e.max() <= 254
    assert abs(np.median(e) - (127 + np.floor(np.log2(0.02 * 0.6745)) - 2)) <= 1
    assert abs(mx[:, :16].mean() - 127.5) < 0.5
    # bf16 rounding is nearest-even: the rounded value is within half a bf16 ulp
    f = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = G.bf16_bits_to_f32(G.f32_to_bf16_bits(f))
    half_ulp = 2.0 ** (np.floor(np.log2(np.abs(f))) - 8)
    assert np.all(np.abs(r - f) <= half_ulp)


def test_zipf_bias_shares_experts_across_verify_tokens():
    w = WORKLOADS["mtp_verify_t4_q2"]
    wr = G.router_weights(1, 0, w.hidden, w.n_experts)
    b = G.router_bias(1, 0, w.n_experts)
    uniq = []
    for s in range(20):
        x = G.bf16_bits_to_f32(np.stack([G.token_candidates(1, s, t, w.hidden) for t in range(4)]))
        _, idx, _, _ = O.route(x.astype(np.float64), wr, b, w.top_k)
        uniq.append(np.unique(idx).size)
    assert 12 <= np.mean(uniq) <= 32          # well below the 40 of disjoint selections


# ------------------------------------------------------------------ planted mistakes
def _tiny():
    H, I, E, k, T, fmt = 64, 32, 5, 2, 3, 3
    wr = G.router_weights(11, 0, H, E)
    b = G.router_bias(11, 0, E)
    recs = [G.expert_canonical(11, 0, e, H, I, fmt) for e in range(E)]
    x = G.bf16_bits_to_f32(np.stack([G.token_candidates(11, 0, t, H) for t in range(T)])).astype(np.float64)
    return H, I, E, k, T, fmt, wr, b, recs, x


def _agrees(H, I, E, k, T, fmt, wr, b, recs, x):
    got, _ = O.moe_layer(x, wr, b, lambda e: recs[e], H, I, k, fmt)
    ref = _dense_reference(x, wr, b, recs, None, H, I, k, fmt, False)
    return np.allclose(got, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_unplanted_oracle_agrees():
    assert _agrees(*_tiny())


@pytest.mark.parametrize("mistake", [
    "offset", "silu_on_up", "no_renorm", "drop_bias", "transpose_down", "bit_order", "k_plus_one"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    args = _tiny()
    if mistake == "offset":
        monkeypatch.setitem(OM.OFFSET, 3, 3.0)
    elif mistake == "silu_on_up":
        real = OM.expert_ffn
        monkeypatch.setattr(OM, "expert_ffn", lambda x, g, u, d: real(x, u, g, d))
    elif mistake == "no_renorm":
        def all_e(logits, idx):
            z = np.exp(logits - logits.max(axis=1, keepdims=True))
            return np.take_along_axis(z / z.sum(axis=1, keepdims=True), idx, axis=1)
        monkeypatch.setattr(OM, "routing_weights", all_e)
    elif mistake == "drop_bias":
        real = OM.router_logits
        monkeypatch.setattr(OM, "router_logits", lambda x, w, b=None: real(x, w, None))
    elif mistake == "transpose_down":
        real = OM.dequant_expert

        def tr(rec, H, I, fmt):
            g, u, d = real(rec, H, I, fmt)
            return g, u, d.reshape(I, H).T.copy()
        monkeypatch.setattr(OM, "dequant_expert", tr)
    elif mistake == "bit_order":
        def msb_first(cb, bits):            # bits read most-significant first
            stream = np.unpackbits(np.asarray(cb, dtype=np.uint8), axis=-1, bitorder="big")
            n = stream.shape[-1] // bits
            stream = stream[..., :n * bits].reshape(*stream.shape[:-1], n, bits).astype(np.int64)
            return (stream * (np.int64(1) << np.arange(bits)[::-1])).sum(axis=-1)
        monkeypatch.setattr(OM, "unpack_codes", msb_first)
    elif mistake == "k_plus_one":
        real = OM.select_topk
        monkeypatch.setattr(OM, "select_topk", lambda l, k: real(l, k + 1))
    assert not _agrees(*args)


# ------------------------------------------------------------------ planted MXFP4 mistakes
def _tiny_mx():
    H, I, E, k, T, fmt = 64, 32, 5, 2, 3, 5
    wr = G.router_weights(12, 0, H, E)
    b = G.router_bias(12, 0, E)
    recs = [G.expert_canonical(12, 0, e, H, I, fmt) for e in range(E)]
    x = G.bf16_bits_to_f32(np.stack([G.token_candidates(12, 0, t, H) for t in range(T)])).astype(np.float64)
    return H, I, E, k, T, fmt, wr, b, recs, x


def test_unplanted_mxfp4_oracle_agrees():
    assert _agrees(*_tiny_mx())


@pytest.mark.parametrize("mistake", ["e2m1_bias", "e2m1_no_subnormal", "e8m0_bias", "sign_bit"])
def test_planted_mxfp4_mistake_is_caught(monkeypatch, mistake):
    args = _tiny_mx()
    if mistake == "e2m1_bias":                  # exponent bias 0 instead of 1
        def v(q):
            q = np.asarray(q, dtype=np.int64)
            ex, m = (q >> 1) & 3, (q & 1).astype(np.float64)
            mag = np.where(ex == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(ex.astype(np.float64)))
            return np.where(q & 8, -1.0, 1.0) * mag
        monkeypatch.setattr(OM, "e2m1_value", v)
    elif mistake == "e2m1_no_subnormal":        # exponent field 0 read as a normal number
        def v(q):
            q = np.asarray(q, dtype=np.int64)
            ex, m = (q >> 1) & 3, (q & 1).astype(np.float64)
            mag = (1.0 + 0.5 * m) * np.exp2(ex.astype(np.float64) - 1.0)
            return np.where(q & 8, -1.0, 1.0) * mag
        monkeypatch.setattr(OM, "e2m1_value", v)
    elif mistake == "e8m0_bias":                # scale 2^(e - 128)
        monkeypatch.setattr(OM, "e8m0_value", lambda e: np.exp2(np.asarray(e, dtype=np.float64) - 128.0))
    elif mistake == "sign_bit":                 # sign taken from bit 0
        real = OM.e2m1_value
        monkeypatch.setattr(OM, "e2m1_value",
                            lambda q: real(((np.asarray(q) & 1) << 3) | (np.asarray(q) & 6) | ((np.asarray(q) >> 3) & 1)))
    assert not _agrees(*args)
