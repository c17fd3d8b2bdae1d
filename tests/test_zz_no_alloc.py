"""The allocation-free entry point (strata_moe_forward_static) against the
workspace one (strata_moe_forward): same kernels, same inputs, so the outputs
must be identical, bit for bit, on two calls in a row on the shared static
array, the second smaller than the first; calls too large for the array are
refused before anything runs."""

import numpy as np
import pytest
import torch

from tests.moe_cases import HostLayer, tokens, to_device_bf16, device_layer

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    from quantized_moe_expert_gemv_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


def _pair(B, layer, x, flags=0):
    T, H = x.shape
    ref = torch.empty((T, H), dtype=torch.float32, device=DEV)
    got = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    B.strata_moe_forward(layer.handle, x, T, ref, flags)
    B.strata_moe_forward_static(layer.handle, x, T, got, flags)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("fmt,shared", [(2, 0), (4, 1)])
@pytest.mark.parametrize("sizes", [(8, 3), (200, 40)])
def test_static_matches_workspace_twice(B, fmt, shared, sizes):
    hl = HostLayer(61, 0, 512, 256, 32, 4, fmt, True, shared)
    layer = device_layer(hl, 256, DEV)
    for i, T in enumerate(sizes):                    # the second call is smaller
        bits, _ = tokens(hl, 500 + 10 * i + T, T)
        x = to_device_bf16(bits, DEV)
        ref, got = _pair(B, layer, x)
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), f"call {i} (T={T}) differs from the workspace entry point"
    # residual flag through the static path too
    bits, _ = tokens(hl, 590, 5)
    x = to_device_bf16(bits, DEV)
    base = torch.linspace(-1, 1, 5 * hl.H, device=DEV).reshape(5, hl.H)
    ref, got = base.clone(), base.clone()
    B.strata_moe_forward(layer.handle, x, 5, ref, B.STRATA_ACCUMULATE)
    B.strata_moe_forward_static(layer.handle, x, 5, got, B.STRATA_ACCUMULATE)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    layer.close()


def test_static_full_size_decode_and_refusal(B):
    """The 2560-wide, 512-expert, top-10 Q2 layer: 4-token and 1-token calls
    through the static array match the workspace path; a call whose regions
    exceed the array is refused with STRATA_E_UNSUPPORTED and leaves the
    output untouched."""
    hl = HostLayer(2026, 0, 2560, 512, 512, 10, 2, True)
    layer = device_layer(hl, 1024, DEV)
    for T in (4, 1):
        bits, _ = tokens(hl, 900 + T, T)
        ref, got = _pair(B, layer, to_device_bf16(bits, DEV))
        assert torch.equal(got, ref)
    big = torch.zeros((1024, hl.H), dtype=torch.bfloat16, device=DEV)
    out = torch.full((1024, hl.H), 7.0, device=DEV)
    with pytest.raises(B.StrataError) as e:
        B.strata_moe_forward_static(layer.handle, big, 1024, out)
    assert e.value.code == B.STRATA_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    layer.close()
