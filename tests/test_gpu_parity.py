"""GPU parity: the HIP path through the C ABI vs the fp64 oracle on the same
seeded inputs.  Routing (ids, permutation, offsets) must be bit-exact; the
fp32 decode path within rel-L2 1e-5; the 16-bit-MFMA prefill path within
rel-L2 2e-2.  Both bounds hold for the call as a whole and for every single
token row compared (check_rows)."""

import os

import numpy as np
import pytest
import torch

import oracle as O
from moe_synth import WORKLOADS, generate as G
from tests.moe_cases import (HostLayer, tokens, to_device_bf16, device_layer, rel_l2, check_route,
                             check_rows, tile_tokens, DECODE_TOL, PREFILL_TOL)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    from quantized_moe_expert_gemv_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


_layers = {}


def tiny(fmt, biased=True, n_shared=0, H=256, I=256, E=16, k=4, max_tokens=320, seed=101):
    key = (fmt, biased, n_shared, H, I, E, k, max_tokens, seed)
    if key not in _layers:
        hl = HostLayer(seed, fmt, H, I, E, k, fmt, biased, n_shared)
        _layers[key] = (hl, device_layer(hl, max_tokens, DEV))
    return _layers[key]


# ------------------------------------------------------------------ small shapes, every format
@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
@pytest.mark.parametrize("T", [1, 3, 8, 9, 13, 16])
def test_decode_route_and_forward_tiny(B, fmt, T):
    hl, layer = tiny(fmt)
    bits, xf = tokens(hl, 10 + T, T)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf)
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, DECODE_TOL, f"decode fmt {fmt} T {T}")


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_decode_two_superblocks_per_wave(B, fmt):
    """H = 3072 (12 superblocks): six gate/up waves of two superblocks each,
    the case whose second superblock's slabs are requested while the first
    computes (1-3 tokens), with the shared expert."""
    hl, layer = tiny(fmt, n_shared=1, H=3072, I=256, E=16, k=4, max_tokens=16)
    for T in (1, 2, 3, 5):
        bits, xf = tokens(hl, 50 + T, T)
        x = to_device_bf16(bits, DEV)
        check_route(layer, hl, x, xf)
        out = layer.forward(x).cpu().numpy()
        ref, _ = hl.oracle(xf)
        check_rows(out, ref, DECODE_TOL, f"decode H 3072 fmt {fmt} T {T}")


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
def test_decode_shared_expert_tiny(B, fmt):
    hl, layer = tiny(fmt, n_shared=1)
    for T in (1, 4, 16):
        bits, xf = tokens(hl, 30 + T, T)
        out = layer.forward(to_device_bf16(bits, DEV)).cpu().numpy()
        ref, _ = hl.oracle(xf)
        check_rows(out, ref, DECODE_TOL, f"decode+shared fmt {fmt} T {T}")


@pytest.mark.parametrize("T", [3, 12, 130])
def test_mxfp4_extreme_scales(B, T):
    """MXFP4 blocks whose E8M0 scale byte is 0 (read as zero by the kernels,
    2^-127 by the oracle: below every tolerance), 1 (2^-126, the smallest
    normal float; zero once rounded to fp16 in the prefill operands) and 127
    (scale 1: weights up to 6, ~300 times the drawn ones), each on about 5%
    of the blocks, through both paths."""
    hl = HostLayer(103, 5, 256, 256, 16, 4, 5, True, 1)
    rng = np.random.default_rng(7)
    for rec in (hl.canon.reshape(hl.E, -1, 17), hl.shared.reshape(1, -1, 17)):
        u = rng.random(rec.shape[:2])
        rec[..., 16] = np.where(u < 0.05, 0, np.where(u < 0.10, 1, np.where(u < 0.15, 127, rec[..., 16])))
    layer = device_layer(hl, 320, DEV)
    bits, xf = tokens(hl, 40 + T, T)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, w_atol=5e-5)
    ref, _ = hl.oracle(xf)
    check_rows(layer.forward(x).cpu().numpy(), ref, DECODE_TOL if T <= 16 else PREFILL_TOL, f"mxfp4 extreme T {T}")


@pytest.mark.parametrize("E,k", [(64, 6), (300, 10), (512, 10), (1024, 8)])
@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_decode_expert_counts(B, E, k, T):
    """Expert counts below, at and above 512 (the top-k kernel's per-wave
    id ranges: 1 to 4 logits per lane, padded ids past E)."""
    hl, layer = tiny(2, E=E, k=k, max_tokens=16)
    bits, xf = tokens(hl, 700 + T, T)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf)
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, DECODE_TOL, f"decode E {E} k {k} T {T}")


def test_decode_lds_limit_falls_back_to_prefill(B):
    """Top-64 of 512 experts at 8 tokens: the decode down kernel's routing
    table and staged rows do not fit in LDS, so the call takes the
    decode kernels of 9..16 tokens (routed rows staged per pass).  Top-300 of
    4096 at 8 tokens (2400 active experts): neither down kernel's routing
    table fits, so the call takes the grouped-GEMM path and forcing decode is
    refused; at 2 tokens (600) the staged kernel holds it."""
    hl, layer = tiny(2, E=512, k=64, max_tokens=16)
    bits, xf = tokens(hl, 950, 8)
    x = to_device_bf16(bits, DEV)
    ref, _ = hl.oracle(xf)
    check_rows(layer.forward(x, flags=B.STRATA_FORCE_DECODE).cpu().numpy(), ref, DECODE_TOL,
               "top-64 T 8 (decode kernels of 9..16 tokens)")
    hl, layer = tiny(2, E=4096, k=300, max_tokens=80)
    bits, xf = tokens(hl, 951, 8)
    x = to_device_bf16(bits, DEV)
    ref, _ = hl.oracle(xf)
    check_route(layer, hl, x, xf, w_atol=5e-5)
    check_rows(layer.forward(x).cpu().numpy(), ref, PREFILL_TOL, "top-300 of 4096 T 8 (grouped path)")
    with pytest.raises(B.StrataError) as e:
        B.strata_moe_forward(layer.handle, x, 8, torch.empty((8, hl.H), device=DEV), B.STRATA_FORCE_DECODE)
    assert e.value.code == B.STRATA_E_UNSUPPORTED
    bits2, xf2 = tokens(hl, 952, 2)
    x2 = to_device_bf16(bits2, DEV)
    check_route(layer, hl, x2, xf2, flags=B.STRATA_FORCE_DECODE, w_atol=5e-5)
    ref2, _ = hl.oracle(xf2)
    check_rows(layer.forward(x2, flags=B.STRATA_FORCE_DECODE).cpu().numpy(), ref2, DECODE_TOL,
               "top-300 of 4096 T 2 (decode)")


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
@pytest.mark.parametrize("T", [1, 9, 130, 300])
def test_prefill_route_and_forward_tiny(B, fmt, T):
    hl, layer = tiny(fmt, n_shared=1 if fmt >= 4 else 0)
    bits, xf = tokens(hl, 50 + T, T)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, flags=B.STRATA_FORCE_PREFILL, w_atol=5e-5)
    out = layer.forward(x, flags=B.STRATA_FORCE_PREFILL).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, PREFILL_TOL, f"prefill fmt {fmt} T {T}")
    # the decode and prefill paths agree per token to the prefill bound
    if T <= 8:
        dec = layer.forward(x).cpu().numpy()
        check_rows(out, dec, PREFILL_TOL, f"prefill vs decode fmt {fmt} T {T}")


def test_prefill_multi_tile_experts(B):
    # few experts, many tokens: every expert spans several 128-row tiles plus a ragged tail
    hl = HostLayer(7, 0, 512, 512, 8, 2, 2, True)
    layer = device_layer(hl, 1000, DEV)
    bits, xf = tokens(hl, 1, 1000)
    x = to_device_bf16(bits, DEV)
    oidx = check_route(layer, hl, x, xf, w_atol=5e-5)
    assert np.bincount(oidx.reshape(-1), minlength=8).max() > 2 * 128
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, PREFILL_TOL, "multi-tile experts T 1000")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fmt", [2, 4])
def test_prefill_many_items_per_workgroup_every_row(B, fmt):
    """16384 tokens over 32 Zipf-skewed experts (H = I = 512, top-4): about
    540 row tiles, so each persistent GEMM workgroup walks several work items
    of every row class (the cross-item prefetch and the per-class loops); every
    output row is compared with the oracle."""
    hl = HostLayer(11, 0, 512, 512, 32, 4, fmt, True)
    layer = device_layer(hl, 16384, DEV)
    bits, xf = tokens(hl, 5, 16384)
    x = to_device_bf16(bits, DEV)
    oidx = check_route(layer, hl, x, xf, w_atol=5e-5)
    counts = np.bincount(oidx.reshape(-1), minlength=hl.E)
    n_tiles = int(np.sum((counts + 127) // 128))
    col_tiles = 512 // (256 if fmt == 2 else 128)
    assert n_tiles * col_tiles > 4 * 256, n_tiles          # several items per workgroup
    assert ((counts % 128) > 0).sum() > 16                  # ragged remainders of every size
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, PREFILL_TOL, f"16K tokens fmt {fmt}")


@pytest.mark.parametrize("T", [64, 300])
def test_prefill_topk_beyond_512_experts(B, T):
    """1024 experts, top-8, through the grouped path (its top-k streams the
    logit row instead of holding it in registers): routing exact, every row
    compared."""
    hl, layer = tiny(2, E=1024, k=8, max_tokens=320)
    bits, xf = tokens(hl, 810 + T, T)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, flags=B.STRATA_FORCE_PREFILL, w_atol=5e-5)
    out = layer.forward(x, flags=B.STRATA_FORCE_PREFILL).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, PREFILL_TOL, f"E 1024 prefill T {T}")


@pytest.mark.parametrize("path", ["decode", "decode16", "prefill"])
def test_exact_ties_and_nan_logits(B, path):
    """Experts 0..7 get zero router rows and the same bias 0.5, so their
    logits tie exactly at 0.5 for every token and the tie straddles rank k:
    equal logits go to the lower expert id.  Expert 13's bias is NaN: a NaN
    logit ranks below every number and is never selected.  Ids, permutation,
    offsets bit-exact and outputs within the path's bound."""
    hl = HostLayer(21, 0, 256, 256, 16, 4, 2, True)
    hl.wr = hl.wr.copy()
    hl.wr[:8] = 0.0
    hl.b = np.zeros(hl.E, dtype=np.float32)
    hl.b[:8] = 0.5
    hl.b[13] = np.nan
    layer = device_layer(hl, 64, DEV)
    T = {"decode": 6, "decode16": 12, "prefill": 40}[path]
    bits, xf = tokens(hl, 77, T, min_gap=0.0)
    l = hl.logits(xf)
    _, oidx, _, _ = O.route(xf, hl.wr, hl.b, hl.k)
    tied = np.isin(oidx, np.arange(8)).sum(axis=1)
    above = (np.nan_to_num(l[:, 8:], nan=-np.inf) > 0.5).sum(axis=1)
    assert np.any((tied > 0) & (above > 0) & (tied < 8))   # ties cut at rank k
    assert not np.any(oidx == 13)
    flags = B.STRATA_FORCE_PREFILL if path == "prefill" else B.STRATA_FORCE_DECODE
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, flags=flags, w_atol=5e-5 if path == "prefill" else 2e-6)
    ref, _ = hl.oracle(xf)
    check_rows(layer.forward(x, flags=flags).cpu().numpy(), ref,
               PREFILL_TOL if path == "prefill" else DECODE_TOL, f"ties {path}")


@pytest.mark.parametrize("fmt", [2, 3, 4, 5])
@pytest.mark.parametrize("H,I", [(96, 160), (2592, 800)])
def test_widths_in_whole_blocks(B, fmt, H, I):
    """Hidden and intermediate widths that are whole 32-weight blocks but not
    whole 256-weight superblocks (zero-padded inside the library): decode and
    grouped paths, with the shared expert and the residual add, every row
    against the oracle."""
    hl = HostLayer(31, 0, H, I, 16, 4, fmt, True, 1 if fmt >= 4 else 0)
    layer = device_layer(hl, 64, DEV)
    for T in (3, 12, 40):
        bits, xf = tokens(hl, 600 + T, T)
        x = to_device_bf16(bits, DEV)
        check_route(layer, hl, x, xf, w_atol=5e-5)
        ref, _ = hl.oracle(xf)
        tol = DECODE_TOL if T <= 16 else PREFILL_TOL
        check_rows(layer.forward(x).cpu().numpy(), ref, tol, f"H {H} I {I} fmt {fmt} T {T}")
        out = torch.zeros((T, H), dtype=torch.float32, device=DEV)
        layer.forward(x, out=out, flags=B.STRATA_ADD_INPUT)
        check_rows(out.cpu().numpy(), ref + xf, tol, f"H {H} I {I} fmt {fmt} T {T} + x")
    if fmt == 2:                            # fp32 tokens through the padded router rows
        xf32 = torch.from_numpy(xf.astype(np.float32)).to(DEV)
        check_rows(layer.forward(xf32).cpu().numpy(), ref, PREFILL_TOL, f"H {H} I {I} fp32 tokens")


@pytest.mark.parametrize("E,k,T,path", [(512, 100, 4, "decode"), (512, 100, 12, "decode"), (512, 100, 40, "prefill"),
                                        (96, 96, 3, "decode"), (96, 96, 50, "prefill"),
                                        (4096, 300, 2, "decode"), (4096, 300, 9, "prefill"),
                                        (1024, 65, 70, "prefill")])
def test_top_k_beyond_64(B, E, k, T, path):
    """Selections past 64 experts per token (block top-k, any k up to E):
    ids, weights, permutation and offsets exact, every output row within the
    path's bound."""
    hl, layer = tiny(2, E=E, k=k, max_tokens=80)
    bits, xf = tokens(hl, 880 + T, T, min_gap=0.0 if k == E else 1e-2)
    x = to_device_bf16(bits, DEV)
    flags = B.STRATA_FORCE_PREFILL if path == "prefill" else B.STRATA_FORCE_DECODE
    check_route(layer, hl, x, xf, flags=flags, w_atol=5e-5)
    ref, _ = hl.oracle(xf)
    check_rows(layer.forward(x, flags=flags).cpu().numpy(), ref, DECODE_TOL if path == "decode" else PREFILL_TOL,
               f"E {E} k {k} T {T} {path}")


@pytest.mark.parametrize("fmt,H,I,n_shared", [(2, 256, 256, 0), (4, 256, 256, 1), (3, 2592, 800, 0)])
@pytest.mark.parametrize("T", [9, 32, 33, 64])
def test_one_launch_route(B, fmt, H, I, n_shared, T):
    """Routing in one launch (router, top-k, permutation; the last workgroup
    routes): ids, weights, permutation and offsets exact, outputs per row
    within the grouped path's bound, identical to the multi-launch routing's
    outputs (up to the logits' summation order), and unchanged over repeated
    calls (the completion counter resets
    itself), bf16 and fp32 tokens; the two routings agree to 1e-5."""
    hl = HostLayer(41, 0, H, I, 32, 4, fmt, True, n_shared)
    layer = device_layer(hl, 64, DEV)
    bits, xf = tokens(hl, 1000 + T, T)
    x = to_device_bf16(bits, DEV)
    fused = B.STRATA_FORCE_PREFILL | B.STRATA_FUSED_ROUTE
    split = B.STRATA_FORCE_PREFILL | B.STRATA_SPLIT_ROUTE
    check_route(layer, hl, x, xf, flags=fused, w_atol=5e-5)
    ref, _ = hl.oracle(xf)
    a = layer.forward(x, flags=fused).clone()
    check_rows(a.cpu().numpy(), ref, PREFILL_TOL, f"one-launch route fmt {fmt} H {H} T {T}")
    b = layer.forward(x, flags=split)
    # same selection and expert GEMMs; the logits are summed in another order
    # (full K per wave, then the waves, against split-K planes), so the weights
    # may differ in the last bits
    check_rows(a.cpu().numpy(), b.cpu().numpy(), 1e-5, "one-launch vs multi-launch routing")
    for _ in range(3):
        assert torch.equal(layer.forward(x, flags=fused), a)
    xf32 = torch.from_numpy(xf.astype(np.float32)).to(DEV)
    check_rows(layer.forward(xf32, flags=fused).cpu().numpy(), ref, PREFILL_TOL, f"one-launch route fp32 T {T}")
    with pytest.raises(B.StrataError) as e:
        B.strata_moe_forward(layer.handle, x, T, torch.empty((T, H), device=DEV), fused | B.STRATA_SPLIT_ROUTE)
    assert e.value.code == B.STRATA_E_INVALID


def test_one_launch_route_refuses_large_calls(B):
    hl, layer = tiny(2, E=1024, k=8, max_tokens=320)
    x = torch.zeros((100, hl.H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.StrataError) as e:
        B.strata_moe_forward(layer.handle, x, 100, torch.empty((100, hl.H), device=DEV), B.STRATA_FUSED_ROUTE)
    assert e.value.code == B.STRATA_E_UNSUPPORTED


@pytest.mark.parametrize("fmt,n_shared", [(2, 0), (5, 1)])
@pytest.mark.parametrize("factor", [1e3, 1e6, 2.0 ** 40])
@pytest.mark.parametrize("T", [1, 3, 6, 12, 40])
def test_tokens_far_beyond_the_fp16_range(B, fmt, n_shared, factor, T):
    """Tokens scaled up to 2^40 (bf16 and fp32): the 16-bit operands hold each
    token times a power of two chosen from its largest magnitude, the
    activations carry its square, and the weights undo both, so decode and
    grouped outputs still match the oracle row by row (the selection of
    such tokens is set by their router logits alone; the bias is negligible
    beside them)."""
    hl, layer = tiny(fmt, n_shared=n_shared)
    bits, xf = tokens(hl, 1300 + T, T)
    xs = xf * factor
    xb = torch.from_numpy(G.f32_to_bf16_bits(xs.astype(np.float32)).astype(np.int16)).to(DEV).view(torch.bfloat16)
    xsb = G.bf16_bits_to_f32(G.f32_to_bf16_bits(xs.astype(np.float32))).astype(np.float64)
    tol = DECODE_TOL if T <= 16 else PREFILL_TOL
    ref, _ = hl.oracle(xsb)
    # ids exact; the router's rounding error grows with the logits (fp32
    # products in decode, bf16 hi/lo products, accurate to about 2^-16, in the
    # grouped path), so near-equal logits of a few thousand move their softmax
    # weights by up to ~1e-5 (decode) or ~1e-4 (grouped)
    check_route(layer, hl, xb, xsb, w_atol=(2e-6 if T <= 16 else 5e-5) * max(1.0, factor / 100))
    # the outputs: against the oracle, and (decode: at its own bound) against
    # the oracle's experts weighted by the device router's weights, which
    # removes the router's rounding from the comparison
    out = layer.forward(xb).cpu().numpy()
    check_rows(out, ref, tol if T > 16 else tol * max(1.0, factor / 100), f"x * {factor:g} bf16 fmt {fmt} T {T}")
    idx, w, _, _ = layer.route(xb)
    check_rows(out, hl.mixture(xsb, idx.cpu().numpy(), w.cpu().numpy()), tol,
               f"x * {factor:g} bf16 fmt {fmt} T {T}, device weights")
    x32 = torch.from_numpy(xs.astype(np.float32)).to(DEV)
    x32f = xs.astype(np.float32).astype(np.float64)
    ref32, _ = hl.oracle(x32f)
    out32 = layer.forward(x32).cpu().numpy()
    check_rows(out32, ref32, tol if T > 16 else tol * max(1.0, factor / 100), f"x * {factor:g} fp32 fmt {fmt} T {T}")
    idx, w, _, _ = layer.route(x32)
    check_rows(out32, hl.mixture(x32f, idx.cpu().numpy(), w.cpu().numpy()), tol,
               f"x * {factor:g} fp32 fmt {fmt} T {T}, device weights")


@pytest.mark.parametrize("fmt", [2, 4])
@pytest.mark.parametrize("T", [2, 4, 6, 12, 40])
def test_mixed_token_scales_in_one_call(B, fmt, T):
    """Tokens of one call at different magnitudes (x1, x1e3, x2^40, x1e-3
    in turn): each takes its own operand scale (decode: found by the router
    kernel up to 4 tokens, by the top-k kernel above; 40 tokens: the grouped
    path), so every row matches the oracle's experts weighted by the device
    router's weights."""
    hl, layer = tiny(fmt)
    bits, xf = tokens(hl, 1700 + T, T)
    f = np.array([1.0, 1e3, 2.0 ** 40, 1e-3])[np.arange(T) % 4][:, None]
    xs = (xf * f).astype(np.float32)
    for x, xd in ((xs.astype(np.float64), torch.from_numpy(xs).to(DEV)),
                  (G.bf16_bits_to_f32(G.f32_to_bf16_bits(xs)).astype(np.float64),
                   torch.from_numpy(G.f32_to_bf16_bits(xs).astype(np.int16)).to(DEV).view(torch.bfloat16))):
        out = layer.forward(xd).cpu().numpy()
        idx, w, _, _ = layer.route(xd)
        check_rows(out, hl.mixture(x, idx.cpu().numpy(), w.cpu().numpy()), DECODE_TOL if T <= 16 else PREFILL_TOL,
                   f"mixed scales fmt {fmt} T {T} {xd.dtype}")


@pytest.mark.parametrize("fmt,scale", [(2, np.inf), (2, np.nan), (2, 40000.0), (3, 20000.0), (4, 8192.0),
                                       (5, 141), (5, 200), (5, 255)])
def test_block_scales_the_operands_cannot_carry_are_refused(B, fmt, scale):
    """A block scale that no 16-bit weight operand can hold (fp16 d NaN,
    infinite or beyond the format's limit; MXFP4 scale byte 255 or above 140)
    makes create fail with STRATA_E_UNSUPPORTED; the limit itself is
    accepted."""
    hl = HostLayer(51, 0, 256, 256, 8, 2, fmt, True)
    canon = hl.canon.reshape(hl.E, -1, 17 if fmt == 5 else 2 + 4 * fmt).copy()
    good = canon.copy()
    if fmt == 5:
        canon[3, 5, 16] = scale
        good[3, 5, 16] = 140
    else:
        canon[3, 5, -2:] = np.array([scale], dtype="<f2").view(np.uint8)
        good[3, 5, -2:] = np.array([{2: 32768.0, 3: 16384.0, 4: 4096.0}[fmt]], dtype="<f2").view(np.uint8)
    cfg = B.make_config(hl.H, hl.I, hl.E, hl.k, 0, fmt, 16)
    wr = torch.from_numpy(hl.wr).to(DEV)
    b = torch.from_numpy(hl.b).to(DEV)
    with pytest.raises(B.StrataError) as e:
        B.StrataMoE(cfg, wr, b, torch.from_numpy(canon.reshape(-1)).to(DEV))
    assert e.value.code == B.STRATA_E_UNSUPPORTED and "scale" in str(e.value)
    B.StrataMoE(cfg, wr, b, torch.from_numpy(good.reshape(-1)).to(DEV)).close()


@pytest.mark.parametrize("flags_name", ["STRATA_ADD_INPUT", "STRATA_ACCUMULATE"])
@pytest.mark.parametrize("T", [2, 12, 40])
def test_residual_flags(B, flags_name, T):
    hl, layer = tiny(3)
    bits, xf = tokens(hl, 70 + T, T)
    x = to_device_bf16(bits, DEV)
    flags = getattr(B, flags_name)
    base = torch.from_numpy(np.linspace(-1, 1, T * hl.H, dtype=np.float32).reshape(T, hl.H)).to(DEV)
    out = base.clone()
    layer.forward(x, out=out, flags=flags)
    ref, _ = hl.oracle(xf)
    ref = ref + (xf if flags_name == "STRATA_ADD_INPUT" else base.cpu().numpy())
    tol = DECODE_TOL if T <= 16 else PREFILL_TOL
    check_rows(out.cpu().numpy(), ref, tol, f"{flags_name} T {T}")


@pytest.mark.parametrize("T", [1, 5, 16, 64])
def test_fp32_activations(B, T):
    hl, layer = tiny(2, n_shared=1)
    rng = np.random.default_rng(T)
    for _ in range(50):                               # keep a clear top-k margin
        xf = rng.standard_normal((T, hl.H)).astype(np.float32)
        _, gap = O.select_topk(hl.logits(xf), hl.k)
        if gap.min() > 1e-2:
            break
        xf[gap <= 1e-2] = rng.standard_normal((int((gap <= 1e-2).sum()), hl.H))
    x = torch.from_numpy(xf).to(DEV)
    ref, _ = hl.oracle(xf.astype(np.float64))
    out = layer.forward(x).cpu().numpy()
    check_rows(out, ref, DECODE_TOL if T <= 16 else PREFILL_TOL, f"fp32 tokens T {T}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_k_equals_E_is_the_dense_mixture(B, path):
    hl = HostLayer(3, 0, 256, 256, 8, 8, 4, True)
    layer = device_layer(hl, 64, DEV)
    bits, xf = tokens(hl, 2, 4, min_gap=0.0)
    flags = B.STRATA_FORCE_PREFILL if path == "prefill" else 0
    out = layer.forward(to_device_bf16(bits, DEV), flags=flags).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, DECODE_TOL if path == "decode" else PREFILL_TOL, f"k = E {path}")


def test_k1_and_tiny_expert_count(B):
    hl = HostLayer(4, 0, 256, 256, 2, 1, 2, False)
    layer = device_layer(hl, 16, DEV)
    bits, xf = tokens(hl, 3, 5)
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf)
    ref, _ = hl.oracle(xf)
    check_rows(layer.forward(x).cpu().numpy(), ref, DECODE_TOL, "k 1 decode")
    check_rows(layer.forward(x, flags=B.STRATA_FORCE_PREFILL).cpu().numpy(), ref, PREFILL_TOL, "k 1 prefill")


@pytest.mark.parametrize("T", [4, 16, 200])
def test_run_to_run_bit_identical(B, T):
    hl, layer = tiny(2)
    bits, _ = tokens(hl, 90 + T, T)
    x = to_device_bf16(bits, DEV)
    a = layer.forward(x).clone()
    b = layer.forward(x).clone()
    assert torch.equal(a, b)


def test_bad_calls_on_a_live_handle(B):
    hl, layer = tiny(2)
    x = torch.zeros((4, hl.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, hl.H), dtype=torch.float32, device=DEV)
    # T > max_tokens: refused by the library itself (raw call) and by the binding
    import ctypes
    rc = B._lib.strata_moe_forward(layer.handle, ctypes.c_void_p(x.data_ptr()), B.STRATA_BF16, 400,
                                   ctypes.c_void_p(out.data_ptr()), 0, None)
    assert rc == B.STRATA_E_INVALID and "max_tokens" in B.strata_moe_last_error()
    with pytest.raises(ValueError):
        B.strata_moe_forward(layer.handle, x, 400, out)
    with pytest.raises(ValueError):                           # out not fp32 / wrong width
        layer.forward(x, out=torch.empty((4, hl.H), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        layer.forward(torch.zeros((4, hl.H - 32), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):                           # a strided view
        layer.forward(torch.zeros((4, 2 * hl.H), dtype=torch.bfloat16, device=DEV)[:, ::2])
    n = B.STRATA_DECODE_MAX_T + 1
    big = torch.zeros((n, hl.H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.StrataError) as e:
        B.strata_moe_forward(layer.handle, big, n, torch.empty((n, hl.H), device=DEV), B.STRATA_FORCE_DECODE)
    assert e.value.code == B.STRATA_E_UNSUPPORTED
    xo = torch.zeros((4, hl.H), dtype=torch.float32, device=DEV)
    with pytest.raises(B.StrataError):
        B.strata_moe_forward(layer.handle, xo, 4, xo)           # x and out overlap


# ------------------------------------------------------------------ full-size workloads
_full = {}


def full_layer(name, max_tokens):
    w = WORKLOADS[name]
    key = (w.hidden, w.inter, w.n_experts, w.top_k, w.fmt, w.biased, w.n_shared, max_tokens)
    if key not in _full:
        _full.clear()
        hl = HostLayer(2026, 0, w.hidden, w.inter, w.n_experts, w.top_k, w.fmt, w.biased, w.n_shared)
        _full[key] = (hl, device_layer(hl, max_tokens, DEV))
    return _full[key]


@pytest.mark.timeout(600)
def test_workload_decode_t1_q2(B):
    w = WORKLOADS["decode_t1_q2"]
    hl = HostLayer(2026, 0, w.hidden, w.inter, w.n_experts, w.top_k, w.fmt, w.biased)
    layer = device_layer(hl, 1, DEV)
    bits, xf = tokens(hl, 1, 8)
    for t in range(8):
        x = to_device_bf16(bits[t:t + 1], DEV)
        check_route(layer, hl, x, xf[t:t + 1])
        out = layer.forward(x).cpu().numpy()
        ref, _ = hl.oracle(xf[t:t + 1])
        check_rows(out, ref, DECODE_TOL, f"1-token decode {t}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mtp_verify_t4_q2", "lookup_verify_t6_q2"])
def test_workload_verify_q2(B, name):
    """Verify windows through the decode path: 1 + 3 MTP drafts and 1 + 5
    prompt-lookup drafts, four batches each."""
    T = WORKLOADS[name].tokens
    hl, layer = full_layer(name, 8192)
    for s in range(4):
        bits, xf = tokens(hl, 100 + s, T)
        x = to_device_bf16(bits, DEV)
        oidx = check_route(layer, hl, x, xf)
        assert np.unique(oidx).size < 40                  # the Zipf bias shares experts
        out = layer.forward(x).cpu().numpy()
        ref, _ = hl.oracle(xf)
        check_rows(out, ref, DECODE_TOL, f"{name} batch {s}")


def against_decode(layer, x, out, tol=PREFILL_TOL, what=""):
    """Every row of a grouped-path output against the decode path on the same
    tokens (8 at a time; the decode path is held to the oracle at 1e-5 by the
    tests above and on the sampled rows of each caller)."""
    from quantized_moe_expert_gemv_amd import binding as Bn
    T = x.shape[0]
    runs = []
    for _ in range(2):                  # twice: the decode path must be bit-identical run to run
        dec = torch.empty((T, out.shape[1]), dtype=torch.float32, device=DEV)
        for t0 in range(0, T, 8):
            n = min(8, T - t0)
            Bn.strata_moe_forward(layer.handle, x[t0:t0 + n], n, dec[t0:t0 + n], Bn.STRATA_FORCE_DECODE)
        runs.append(dec.cpu().numpy())
    dec = runs[0]
    assert np.array_equal(runs[0], runs[1]), f"{what}: decode path differs between two runs"
    check_rows(out, dec, tol, f"{what} vs decode path")
    return dec


@pytest.mark.timeout(900)
def test_workload_prefill_t8192_q2(B):
    """The 8192-token chunk: routing exact for every token, every output row
    against the oracle."""
    hl, layer = full_layer("prefill_t8192_q2", 8192)
    bits, xf = tokens(hl, 7, 8192)
    x = to_device_bf16(bits, DEV)
    oidx = check_route(layer, hl, x, xf, w_atol=5e-5)
    counts = np.bincount(oidx.reshape(-1), minlength=hl.E)
    assert (counts == 0).sum() > 0                          # some experts get no tokens
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, PREFILL_TOL, "8K chunk")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["skinny_t16_q2", "skinny_t32_q2", "skinny_t64_q2"])
def test_workload_skinny_q2(B, name):
    """Skinny batches (16-64 tokens) of the verify/prefill layer: 16 tokens
    take the decode kernels (one pass over the weights), more the
    grouped-GEMM path with tiles of a few rows; routing exact for every
    token, every output row against the oracle; the grouped path (both
    routings) also at 16 tokens."""
    T = WORKLOADS[name].tokens
    hl, layer = full_layer(name, 8192)
    bits, xf = tokens(hl, 300 + T, T)
    x = to_device_bf16(bits, DEV)
    decode = T <= B.STRATA_DECODE_MAX_T
    check_route(layer, hl, x, xf, w_atol=2e-6 if decode else 5e-5)
    out = layer.forward(x).cpu().numpy()
    ref, _ = hl.oracle(xf)
    check_rows(out, ref, DECODE_TOL if decode else PREFILL_TOL, name)
    # both routings of the grouped path, at the full layer shape
    pre = B.STRATA_FORCE_PREFILL
    check_route(layer, hl, x, xf, flags=pre | B.STRATA_FUSED_ROUTE, w_atol=5e-5)
    check_route(layer, hl, x, xf, flags=pre | B.STRATA_SPLIT_ROUTE, w_atol=5e-5)
    fused = layer.forward(x, flags=pre | B.STRATA_FUSED_ROUTE).cpu().numpy()
    check_rows(fused, ref, PREFILL_TOL, name + " one-launch route")
    check_rows(fused, layer.forward(x, flags=pre | B.STRATA_SPLIT_ROUTE).cpu().numpy(), 1e-5,
               name + " fused vs split")


@pytest.mark.timeout(900)
def test_workload_prefill_t32768_q2(B):
    """The 32768-token chunk: four times the rows per expert of the 8K chunk
    (327,680 token-expert pairs); routing exact for every token, outputs
    compared on a token of every row tile (a random row and the last row of
    each 128-slot tile of every expert: ~2,800 tokens) against the oracle, and
    on every token against the decode path."""
    hl, layer = full_layer("prefill_t32768_q2", 32768)
    bits, xf = tokens(hl, 17, 32768)
    x = to_device_bf16(bits, DEV)
    oidx = check_route(layer, hl, x, xf, w_atol=5e-5)
    counts = np.bincount(oidx.reshape(-1), minlength=hl.E)
    assert counts.max() > 8 * 128                          # the hottest expert spans many row tiles
    out = layer.forward(x).cpu().numpy()
    sample = tile_tokens(oidx, hl.E)
    assert sample.size > 2000
    ref, _ = hl.oracle(xf[sample])
    check_rows(out[sample], ref, PREFILL_TOL, "32K chunk, one token per tile")
    dec = against_decode(layer, x, out, what="32K chunk")
    check_rows(dec[sample[:64]], ref[:64], DECODE_TOL, "32K decode path")


@pytest.mark.timeout(900)
def test_workload_deepseek_q4(B):
    hl, layer = full_layer("deepseek_q4_t2048", 2048)
    bits, xf = tokens(hl, 11, 2048)
    # T = 1 decode
    x1 = to_device_bf16(bits[:1], DEV)
    check_route(layer, hl, x1, xf[:1])
    ref1, _ = hl.oracle(xf[:1])
    check_rows(layer.forward(x1).cpu().numpy(), ref1, DECODE_TOL, "deepseek q4 T 1")
    # T = 2048 prefill: routing exact for every token; sampled rows against
    # the oracle, every row against the decode path
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, w_atol=5e-5)
    out = layer.forward(x).cpu().numpy()
    sample = np.random.default_rng(1).choice(2048, 8, replace=False)
    ref, _ = hl.oracle(xf[sample])
    check_rows(out[sample], ref, PREFILL_TOL, "deepseek q4 2048")
    dec = against_decode(layer, x, out, what="deepseek q4 2048")
    check_rows(dec[sample], ref, DECODE_TOL, "deepseek q4 decode path")


@pytest.mark.timeout(900)
def test_workload_deepseek_mxfp4(B):
    """MXFP4 experts (E2M1 codes, one E8M0 scale per 32 weights) at the
    DeepSeek-shaped layer with its shared expert: one decode token and a
    2048-token prefill."""
    hl, layer = full_layer("deepseek_mxfp4_t2048", 2048)
    bits, xf = tokens(hl, 13, 2048)
    for t in range(2):
        x1 = to_device_bf16(bits[t:t + 1], DEV)
        check_route(layer, hl, x1, xf[t:t + 1])
        ref1, _ = hl.oracle(xf[t:t + 1])
        check_rows(layer.forward(x1).cpu().numpy(), ref1, DECODE_TOL, f"deepseek mxfp4 T 1 ({t})")
    x = to_device_bf16(bits, DEV)
    check_route(layer, hl, x, xf, w_atol=5e-5)
    out = layer.forward(x).cpu().numpy()
    sample = np.random.default_rng(2).choice(2048, 8, replace=False)
    ref, _ = hl.oracle(xf[sample])
    check_rows(out[sample], ref, PREFILL_TOL, "deepseek mxfp4 2048")
    dec = against_decode(layer, x, out, what="deepseek mxfp4 2048")
    check_rows(dec[sample], ref, DECODE_TOL, "deepseek mxfp4 decode path")


# ------------------------------------------------------------------ HIP graph capture and replay
@pytest.mark.parametrize("T,flags", [(1, 0), (4, 0), (16, 0), (100, 0), (40, 16)])
def test_graph_replay_matches_eager(B, T, flags):
    hl, layer = tiny(2, n_shared=1)
    batches = [to_device_bf16(tokens(hl, 200 + 10 * T + i, T)[0], DEV) for i in range(3)]
    eager = [layer.forward(x, flags=flags).clone() for x in batches]
    outs = [torch.empty_like(e) for e in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for x, o in zip(batches, outs):
            layer.forward(x, out=o, flags=flags)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, o in zip(batches, outs):
            layer.forward(x, out=o, flags=flags)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from eager"
        # eager work on the same handle between replays
        layer.forward(batches[rep % 3], flags=flags)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,n_kernels", [(4, 4), (16, 4), (20, 5), (100, 8)])
def test_trace_events_bracket_each_kernel(B, T, n_kernels):
    """Traced calls give the same output and a positive duration per kernel;
    an odd event count is refused."""
    hl, layer = tiny(3)
    x = to_device_bf16(tokens(hl, 300 + T, T)[0], DEV)
    ref = layer.forward(x).clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_kernels)]
    B.strata_moe_trace_next_call(layer.handle, evs)
    out = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for j in range(n_kernels):
        assert evs[2 * j].elapsed_time(evs[2 * j + 1]) > 0.0
    with pytest.raises(B.StrataError):
        B.strata_moe_trace_next_call(layer.handle, evs[:3])


# ------------------------------------------------------------------ stack driver vs chained layer calls
@pytest.mark.parametrize("fmt", [2, 3, 4])
@pytest.mark.parametrize("T", [1, 2])
def test_stack_matches_chained_layer_calls(B, fmt, T):
    """The stack driver (whose single-token 2/3-bit layers also prefetch the
    next layer's router rows and their down slabs) gives exactly what the
    same layers give one call at a time, each adding its input; the first
    layer's own output is also checked against the oracle."""
    hls = [HostLayer(211, l, 256, 512, 16, 4, fmt, True) for l in range(4)]
    layers = [device_layer(hl, 16, DEV) for hl in hls]
    bits, xf = tokens(hls[0], 7, T)
    x = to_device_bf16(bits, DEV)
    h = B.stack_forward(layers, x)
    cur = x
    for layer in layers:
        cur = layer.forward(cur, flags=B.STRATA_ADD_INPUT)
    torch.cuda.synchronize()
    assert torch.equal(h, cur), (h - cur).abs().max().item()
    y1 = layers[0].forward(x).cpu().numpy().astype(np.float64)
    ref, _ = hls[0].oracle(xf)
    assert rel_l2(y1, ref) <= DECODE_TOL
    for layer in layers:
        layer.close()


# ------------------------------------------------------------------ 48-layer Q3 stack (full size)
@pytest.mark.timeout(900)
def test_workload_stack48_q3(B):
    """Every layer resident (42.5 GB), tokens and expected h_48 from the
    oracle (tests/golden/stack48_q3_expected.npz, written by
    tests/golden/make_stack48_expected.py); gated on h_48 - h_0."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "stack48_q3_expected.npz")
    ref = np.load(path)
    w = WORKLOADS["stack48_q3_decode"]
    seed = int(ref["draw"][0][0])
    cfg = B.make_config(w.hidden, w.inter, w.n_experts, w.top_k, 0, w.fmt, 1)
    layers = []
    for l in range(w.n_layers):
        wr = torch.from_numpy(G.router_weights(seed, l, w.hidden, w.n_experts)).to(DEV)
        b = torch.from_numpy(G.router_bias(seed, l, w.n_experts, w.zipf_s)).to(DEV)
        canon = torch.from_numpy(
            G.layer_canonical(seed, l, w.hidden, w.inter, w.n_experts, w.fmt, w.d_sigma).reshape(-1)).to(DEV)
        layers.append(B.StrataMoE(cfg, wr, b, canon))
        del canon
    torch.cuda.synchronize()
    for s in range(ref["x_bits"].shape[0]):
        bits = ref["x_bits"][s:s + 1]
        x = to_device_bf16(bits, DEV)
        h = B.stack_forward(layers, x).cpu().numpy().astype(np.float64)
        x0 = G.bf16_bits_to_f32(bits).astype(np.float64)
        err = rel_l2(h - x0, ref["h48"][s:s + 1] - x0)
        print(f"stack step {s}: rel-L2 of h48 - h0 = {err:.3e}", flush=True)
        assert err <= DECODE_TOL, err
    del layers
    torch.cuda.empty_cache()
