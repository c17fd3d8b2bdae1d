"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, sizes its buffers as documented, and
rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "strata_moe.h")
LIB = os.path.join(ROOT, "quantized_moe_expert_gemv_amd", "libstrata_moe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"STRATA_API\s+[\w\s\*]+?\b(strata_moe_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def B():
    from quantized_moe_expert_gemv_amd import binding
    return binding


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == {"strata_moe_expert_bytes", "strata_moe_packed_bytes",
                          "strata_moe_workspace_bytes", "strata_moe_create", "strata_moe_route",
                          "strata_moe_forward", "strata_moe_forward_static", "strata_moe_stack_forward", "strata_moe_trace_next_call",
                          "strata_moe_destroy", "strata_moe_last_error"}


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == set(declared_functions())


def _cfg(B, **kw):
    base = dict(hidden=2560, inter=512, n_experts=512, top_k=10, n_shared=0, qfmt=2, max_tokens=8)
    base.update(kw)
    return B.make_config(**base)


def test_expert_bytes_match_the_block_format(B):
    # 3 matrices * I * H/32 blocks * (code bytes + 2 scale bytes)
    assert B.strata_moe_expert_bytes(_cfg(B)) == 1228800
    assert B.strata_moe_expert_bytes(_cfg(B, qfmt=3)) == 1720320
    assert B.strata_moe_expert_bytes(_cfg(B, hidden=4096, inter=2048, n_experts=256, top_k=6, qfmt=4)) == 14155776
    # MXFP4 (OCP MX v1.0): 16 bytes of E2M1 codes + one E8M0 scale byte per block
    assert B.strata_moe_expert_bytes(_cfg(B, hidden=7168, inter=2048, n_experts=256, top_k=8, qfmt=5)) == \
        3 * 2048 * (7168 // 32) * 17


def test_mxfp4_packed_bytes_widen_the_scale_to_a_16_bit_slot(B):
    c = _cfg(B, hidden=7168, inter=2048, n_experts=256, top_k=8, qfmt=5)
    blocks = 3 * 2048 * (7168 // 32)
    assert B.strata_moe_packed_bytes(c) >= 256 * blocks * 18 + 2 * 256 * 7168 * 2


def test_packed_bytes_cover_experts_and_router_split(B):
    c = _cfg(B, n_shared=1)
    per = B.strata_moe_expert_bytes(c)
    assert B.strata_moe_packed_bytes(c) >= 513 * per + 2 * 512 * 2560 * 2


def test_workspace_grows_with_max_tokens(B):
    small = B.strata_moe_workspace_bytes(_cfg(B, max_tokens=1))
    big = B.strata_moe_workspace_bytes(_cfg(B, max_tokens=8192))
    # per-pair bf16 expert outputs dominate: 8192 * 10 * 2560 * 2 bytes
    assert small > 0 and big > 8192 * 10 * 2560 * 2 > small


@pytest.mark.parametrize("good", [dict(hidden=2592, inter=800), dict(hidden=32, inter=32, n_experts=4, top_k=4),
                                  dict(top_k=512), dict(n_experts=4096, top_k=4096, max_tokens=4),
                                  dict(hidden=7168, inter=2048, n_experts=256, top_k=8, qfmt=5)])
def test_block_multiples_and_any_k_up_to_e_are_accepted(B, good):
    """Hidden and intermediate widths only need whole 32-weight blocks, and
    top_k may be anything in [1, E]."""
    c = _cfg(B, **good)
    assert B.strata_moe_expert_bytes(c) == 3 * c.inter * (c.hidden // 32) * (17 if c.qfmt == 5 else 2 + 4 * c.qfmt)
    assert B.strata_moe_packed_bytes(c) >= c.n_experts * B.strata_moe_expert_bytes(c)
    assert B.strata_moe_workspace_bytes(c) > 0


@pytest.mark.parametrize("bad", [dict(qfmt=6), dict(qfmt=1), dict(hidden=2500), dict(hidden=2576), dict(inter=100),
                                 dict(inter=48), dict(top_k=0), dict(top_k=513), dict(top_k=101, n_experts=100),
                                 dict(n_experts=0), dict(n_experts=5000), dict(n_shared=2), dict(max_tokens=0),
                                 # one packed Q4 expert past 2 GiB (32-bit offsets inside a record)
                                 dict(hidden=65536, inter=65536, qfmt=4, max_tokens=1)])
def test_invalid_configs_are_rejected(B, bad):
    c = _cfg(B, **bad)
    assert B.strata_moe_packed_bytes(c) == 0
    assert B.strata_moe_workspace_bytes(c) == 0
    h = ctypes.c_void_p()
    dummy = ctypes.c_void_p(256)
    rc = B._lib.strata_moe_create(ctypes.byref(c), dummy, None, dummy, None, dummy, dummy, None,
                                  ctypes.byref(h))
    assert rc in (B.STRATA_E_INVALID, B.STRATA_E_UNSUPPORTED)
    assert h.value is None
    assert B.strata_moe_last_error() != ""


def test_create_rejects_missing_or_misaligned_buffers(B):
    c = _cfg(B)
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(4096)
    rc = B._lib.strata_moe_create(ctypes.byref(c), None, None, p, None, p, p, None, ctypes.byref(h))
    assert rc == B.STRATA_E_INVALID and "non-NULL" in B.strata_moe_last_error()
    rc = B._lib.strata_moe_create(ctypes.byref(c), p, None, p, None, ctypes.c_void_p(4096 + 16), p, None,
                                  ctypes.byref(h))
    assert rc == B.STRATA_E_INVALID and "aligned" in B.strata_moe_last_error()
    rc = B._lib.strata_moe_create(ctypes.byref(c), p, None, p, p, p, p, None, ctypes.byref(h))
    assert rc == B.STRATA_E_INVALID and "shared" in B.strata_moe_last_error()


def test_calls_on_null_handle_fail_cleanly(B):
    rc = B._lib.strata_moe_forward(None, ctypes.c_void_p(256), 0, 1, ctypes.c_void_p(512), 0, None)
    assert rc == B.STRATA_E_INVALID and "handle" in B.strata_moe_last_error()
    rc = B._lib.strata_moe_stack_forward(None, 0, None, 0, 1, None, None, None)
    assert rc == B.STRATA_E_INVALID
    rc = B._lib.strata_moe_trace_next_call(None, None, 0)
    assert rc == B.STRATA_E_INVALID
    B.strata_moe_destroy(None)            # NULL-safe


def test_binding_checks_tensors_before_the_library(B):
    """The binding refuses, before any library call, tensors whose dtype,
    shape, layout or byte size would let the kernels read or write past an
    allocation (checked here on host tensors)."""
    import torch
    cpu = torch.device("cpu")
    B.check_tensor(torch.zeros(4, 8), "t", (4, 8), (torch.float32,), cpu, 128)
    B.check_tensor(torch.zeros(4, 8), "t", (None, 8), (torch.float32,), cpu)
    bad = [
        dict(t=torch.zeros(4, 8, dtype=torch.bfloat16), dtypes=(torch.float32,)),      # dtype
        dict(t=torch.zeros(4, 7), shape=(4, 8)),                                        # width
        dict(t=torch.zeros(3, 8), shape=(4, 8)),                                        # rows
        dict(t=torch.zeros(4, 8, 1), shape=(4, 8)),                                     # rank
        dict(t=torch.zeros(8, 4).t(), shape=(4, 8)),                                    # not contiguous
        dict(t=torch.zeros(4, 8), nbytes=64),                                           # byte size
        dict(t=torch.zeros(4, 8), device=torch.device("meta")),                         # device
        dict(t=[0.0] * 8),                                                              # not a tensor
    ]
    for kw in bad:
        t = kw.pop("t")
        with pytest.raises(ValueError):
            B.check_tensor(t, "t", **kw)
    # the call helpers: x must be on the HIP device, T within max_tokens
    with pytest.raises(ValueError):
        B.strata_moe_forward(None, torch.zeros(2, 256, dtype=torch.bfloat16), 2, torch.zeros(2, 256))
    with pytest.raises(ValueError):
        B._check_call_tensors(torch.zeros(9, 256, dtype=torch.bfloat16), 9, None, 256, 8, cpu)
    with pytest.raises(ValueError):
        B._check_call_tensors(torch.zeros(2, 256, dtype=torch.float16), 2, None, 256, 8, cpu)
