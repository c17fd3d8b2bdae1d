"""ctypes binding of libstrata_moe.so (argument marshalling only).

The functions keep the C names.  Tensors are PyTorch tensors on the HIP
device; only their data pointers, sizes and the current stream cross the
boundary.  Every computation happens in the library's HIP kernels: if the
library is not built, importing this module raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstrata_moe.so")

STRATA_OK, STRATA_E_INVALID, STRATA_E_UNSUPPORTED, STRATA_E_HIP = 0, -1, -2, -3
STRATA_Q2, STRATA_Q3, STRATA_Q4, STRATA_MXFP4 = 2, 3, 4, 5
STRATA_BF16, STRATA_FP32 = 0, 1
STRATA_ACCUMULATE, STRATA_ADD_INPUT, STRATA_FORCE_DECODE, STRATA_FORCE_PREFILL = 1, 2, 4, 8
STRATA_FUSED_ROUTE, STRATA_SPLIT_ROUTE = 16, 32
STRATA_DECODE_MAX_T = 16
STRATA_FUSED_ROUTE_DEFAULT_T = 0

EXPORTS = ("strata_moe_expert_bytes", "strata_moe_packed_bytes", "strata_moe_workspace_bytes",
           "strata_moe_create", "strata_moe_route", "strata_moe_forward",
           "strata_moe_forward_static", "strata_moe_stack_forward", "strata_moe_trace_next_call", "strata_moe_destroy",
           "strata_moe_last_error")
STRATA_MAX_TRACE_EVENTS = 16
STRATA_STATIC_SCRATCH_BYTES = 16 << 20


class strata_moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("qfmt", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32)]


class StrataError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"strata_moe error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_moe_expert_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    cfgp = ctypes.POINTER(strata_moe_config)
    sig = {
        "strata_moe_expert_bytes": (SZ, [cfgp]),
        "strata_moe_packed_bytes": (SZ, [cfgp]),
        "strata_moe_workspace_bytes": (SZ, [cfgp]),
        "strata_moe_create": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, ctypes.POINTER(P)]),
        "strata_moe_route": (ctypes.c_int, [P, P, I32, I32, P, P, P, P, U32, P]),
        "strata_moe_forward": (ctypes.c_int, [P, P, I32, I32, P, U32, P]),
        "strata_moe_forward_static": (ctypes.c_int, [P, P, I32, I32, P, U32, P]),
        "strata_moe_stack_forward": (ctypes.c_int, [ctypes.POINTER(P), I32, P, I32, I32, P, P, P]),
        "strata_moe_trace_next_call": (ctypes.c_int, [P, ctypes.POINTER(P), I32]),
        "strata_moe_destroy": (None, [P]),
        "strata_moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def _check(rc):
    if rc != STRATA_OK:
        raise StrataError(rc, _lib.strata_moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(x):
    if x.dtype == torch.bfloat16:
        return STRATA_BF16
    if x.dtype == torch.float32:
        return STRATA_FP32
    raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")


def check_tensor(t, name, shape=None, dtypes=None, device=None, nbytes=None):
    """Raise ValueError unless t is a contiguous tensor of one of `dtypes`
    with the given shape (None entries match anything), on `device`, of
    `nbytes` bytes.  The library sees only data pointers, so a wrong
    argument here would read or write past an allocation."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and w != g for w, g in zip(shape, t.shape)):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if nbytes is not None and t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{name} must hold {nbytes} bytes, got {t.numel() * t.element_size()}")


def _check_call_tensors(x, T, out=None, hidden=None, max_tokens=None, device=None):
    if T < 1 or (max_tokens is not None and T > max_tokens):
        raise ValueError(f"T = {T} outside [1, {max_tokens}]")
    check_tensor(x, "x", (T, hidden), (torch.bfloat16, torch.float32), device if device is not None else None)
    if device is None and x.device.type != "cuda":
        raise ValueError(f"x must be on the HIP device, got {x.device}")
    if out is not None:
        check_tensor(out, "out", (T, x.shape[1]), (torch.float32,), x.device)


def make_config(hidden, inter, n_experts, top_k, n_shared, qfmt, max_tokens):
    return strata_moe_config(hidden, inter, n_experts, top_k, n_shared, qfmt, max_tokens)


def strata_moe_expert_bytes(cfg):
    return _lib.strata_moe_expert_bytes(ctypes.byref(cfg))


def strata_moe_packed_bytes(cfg):
    return _lib.strata_moe_packed_bytes(ctypes.byref(cfg))


def strata_moe_workspace_bytes(cfg):
    return _lib.strata_moe_workspace_bytes(ctypes.byref(cfg))


def strata_moe_create(cfg, router_w, router_bias, experts_canon, shared_canon, packed, workspace,
                      stream=None):
    """Returns the opaque handle (a ctypes void pointer)."""
    h = ctypes.c_void_p()
    _check(_lib.strata_moe_create(ctypes.byref(cfg), _ptr(router_w), _ptr(router_bias),
                                  _ptr(experts_canon), _ptr(shared_canon), _ptr(packed),
                                  _ptr(workspace), _stream(stream), ctypes.byref(h)))
    return h


def strata_moe_route(h, x, T, topk_idx, topk_w, perm, offsets, flags=0, stream=None):
    _check_call_tensors(x, T)
    check_tensor(topk_idx, "topk_idx", (T, None), (torch.int32,), x.device)
    k = topk_idx.shape[1]
    check_tensor(topk_w, "topk_w", (T, k), (torch.float32,), x.device)
    check_tensor(perm, "perm", (T * k,), (torch.int32,), x.device)
    check_tensor(offsets, "offsets", (None,), (torch.int32,), x.device)
    _check(_lib.strata_moe_route(h, _ptr(x), _dtype_code(x), T, _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(perm), _ptr(offsets), flags, _stream(stream)))


def strata_moe_forward(h, x, T, out, flags=0, stream=None):
    _check_call_tensors(x, T, out)
    _check(_lib.strata_moe_forward(h, _ptr(x), _dtype_code(x), T, _ptr(out), flags, _stream(stream)))


def strata_moe_forward_static(h, x, T, out, flags=0, stream=None):
    _check_call_tensors(x, T, out)
    _check(_lib.strata_moe_forward_static(h, _ptr(x), _dtype_code(x), T, _ptr(out), flags, _stream(stream)))


def strata_moe_stack_forward(handles, x, T, out, tmp, stream=None):
    _check_call_tensors(x, T, out)
    check_tensor(tmp, "tmp", tuple(out.shape), (torch.float32,), x.device)
    arr = (ctypes.c_void_p * len(handles))(*[h.value for h in handles])
    _check(_lib.strata_moe_stack_forward(arr, len(handles), _ptr(x), _dtype_code(x), T, _ptr(out),
                                         _ptr(tmp), _stream(stream)))


def strata_moe_trace_next_call(h, events):
    """Arm per-kernel timing of the next call with torch.cuda.Event objects
    (enable_timing=True).  Each event is recorded once first so that its HIP
    event exists."""
    handles = []
    for ev in events:
        if ev.cuda_event == 0:
            ev.record()
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(_lib.strata_moe_trace_next_call(h, arr, len(handles)))


def strata_moe_destroy(h):
    _lib.strata_moe_destroy(h)


def strata_moe_last_error():
    return _lib.strata_moe_last_error().decode()


class StrataMoE:
    """One MoE layer: owns its packed weights and workspace (torch buffers)."""

    def __init__(self, cfg, router_w, router_bias, experts_canon, shared_canon=None, stream=None):
        dev = router_w.device
        if dev.type != "cuda":
            raise ValueError(f"router_w must be on the HIP device, got {dev}")
        E, H = cfg.n_experts, cfg.hidden
        rec = strata_moe_expert_bytes(cfg)
        if rec == 0:
            raise StrataError(STRATA_E_INVALID, strata_moe_last_error())
        check_tensor(router_w, "router_w", (E, H), (torch.float32,), dev)
        if router_bias is not None:
            check_tensor(router_bias, "router_bias", (E,), (torch.float32,), dev)
        check_tensor(experts_canon, "experts_canon", None, None, dev, E * rec)
        if cfg.n_shared:
            if shared_canon is None:
                raise ValueError("n_shared = 1 needs shared_canon")
            check_tensor(shared_canon, "shared_canon", None, None, dev, rec)
        elif shared_canon is not None:
            raise ValueError("shared_canon given but n_shared = 0")
        self.device = dev
        self.cfg = cfg
        self.router_w = router_w.contiguous()
        self.router_bias = None if router_bias is None else router_bias.contiguous()
        self.packed = torch.empty(strata_moe_packed_bytes(cfg), dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(strata_moe_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        self.handle = strata_moe_create(cfg, self.router_w, self.router_bias, experts_canon,
                                        shared_canon, self.packed, self.workspace, stream)

    def route(self, x, flags=0, stream=None):
        T = x.shape[0]
        _check_call_tensors(x, T, None, self.cfg.hidden, self.cfg.max_tokens, self.device)
        k, E = self.cfg.top_k, self.cfg.n_experts
        dev = x.device
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        strata_moe_route(self.handle, x, T, idx, w, perm, offsets, flags, stream)
        return idx, w, perm, offsets

    def forward(self, x, out=None, flags=0, stream=None):
        T = x.shape[0]
        _check_call_tensors(x, T, None, self.cfg.hidden, self.cfg.max_tokens, self.device)
        if out is None:
            out = torch.empty((T, self.cfg.hidden), dtype=torch.float32, device=x.device)
        strata_moe_forward(self.handle, x, T, out, flags, stream)
        return out

    __call__ = forward

    def close(self):
        if self.handle is not None:
            strata_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stack_forward(layers, x, out=None, tmp=None, stream=None):
    if not layers:
        raise ValueError("need at least one layer")
    T = x.shape[0]
    H = layers[0].cfg.hidden
    for l in layers:
        if l.cfg.hidden != H:
            raise ValueError("every layer of a stack must have the same hidden width")
        _check_call_tensors(x, T, None, H, l.cfg.max_tokens, l.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if tmp is None:
        tmp = torch.empty((T, H), dtype=torch.float32, device=x.device)
    strata_moe_stack_forward([l.handle for l in layers], x, T, out, tmp, stream)
    return out
