"""Python binding of libmoe.so: the MoE layer (forward, backward, routing variants) on MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the library's HIP
kernels; this module passes torch tensors' device pointers and the current
stream through the C ABI declared in include/moe.h, with the same names and
argument order.  PyTorch provides device memory and streams.

Importing fails loudly if the library has not been built
(``python routing_dispatch_expert_router_amd/build.py``).
"""
import ctypes
import os

# One HIP runtime per process.  torch ships its own libamdhip64 (same soname,
# libamdhip64.so.7, but requested by torch under the unversioned name): if
# libmoe.so were loaded first, it would bring in /opt/rocm's copy and torch
# would then load a second one, and the two runtimes do not share the device.
# Importing torch first makes libmoe.so bind to torch's runtime.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # plain ctypes use without torch: /opt/rocm's runtime
    _torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
# struct layout version of include/moe.h (MOE_ABI_VERSION); the loader refuses a library built with another
MOE_ABI_VERSION = 1
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_RELU, MOE_ACT_SWIGLU = 0, 1
MOE_DROP_NONE, MOE_DROP_CAPACITY, MOE_DROP_AFFINITY = 0, 1, 2
MOE_ROUTE_TOKEN_CHOICE, MOE_ROUTE_EXPERT_CHOICE = 0, 1
MOE_LOGITS_COMPUTE, MOE_LOGITS_COMPUTE_STORE, MOE_LOGITS_LOAD = 0, 1, 2

CONFIG_FIELDS = ["T", "d_model", "n_heads", "d_head", "n_experts", "top_k", "n_groups", "topk_groups",
                 "renorm", "drop", "capacity", "keep_num", "keep_den", "d_ff", "act", "n_shared",
                 "latent_proj", "residual", "act_dtype", "router_dtype", "route_mode", "sel_bias_gate",
                 "seq_len"]
# fields an older config object may lack: they default to 0 (token choice, no bias in the gate, off)
_OPTIONAL_FIELDS = {"route_mode", "sel_bias_gate", "seq_len"}

# exported symbols, as declared in include/moe.h
SYMBOLS = ["moe_workspace_bytes", "moe_rows_upper_bound", "moe_status_str", "moe_abi_version", "moe_check_config",
           "moe_route", "moe_route_ex", "moe_dispatch", "moe_dispatch_noalloc", "moe_check_topk", "moe_expert_ffn", "moe_expert_ffn_gather", "moe_combine", "moe_layer_fwd",
           "moe_sel_bias_update", "moe_backward_workspace_bytes", "moe_transpose_weights", "moe_layer_bwd"]


class MoeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in CONFIG_FIELDS]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "router_bias", "w1", "w3", "w2", "ws1", "ws3", "ws2", "w_in", "w_out", "sel_bias")]


class MoeLayerIO(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("logits_mode", ctypes.c_int32),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("demand", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("row_of", ctypes.c_void_p),
                ("src_of", ctypes.c_void_p), ("aux_loss", ctypes.c_void_p), ("seq_loss", ctypes.c_void_p),
                ("z", ctypes.c_void_p),
                ("x_perm", ctypes.c_void_p), ("y_perm", ctypes.c_void_p), ("shared_out", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("gu", ctypes.c_void_p)]


class MoeWeightsT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w13t", "w2t", "ws13t", "ws2t", "w_in_t", "w_out_t")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_router", "dbias", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2",
                                                "dw_in", "dw_out")]


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python routing_dispatch_expert_router_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(MoeConfig)
    sig = {
        "moe_workspace_bytes": (S, [Z]),
        "moe_rows_upper_bound": (ctypes.c_int64, [Z]),
        "moe_status_str": (ctypes.c_char_p, [I]),
        "moe_abi_version": (ctypes.c_int32, []),
        "moe_check_config": (I, [Z]),
        "moe_route": (I, [Z, P, P, P, P, I, P, P, P, P, S, P]),
        "moe_route_ex": (I, [Z, P, P, P, P, P, I, P, P, P, P, P, S, P]),
        "moe_sel_bias_update": (I, [Z, P, P, ctypes.c_float, P]),
        "moe_dispatch": (I, [Z, P, P, P, P, P, P, P, P, P, P, S, P]),
        "moe_dispatch_noalloc": (I, [Z, P, P, P, P, P, P, P, P, P, P]),
        "moe_check_topk": (I, [Z, P, P, P]),
        "moe_expert_ffn": (I, [Z, P, P, P, P, P, P, P, P, P, P, P, P, S, P]),
        "moe_expert_ffn_gather": (I, [Z, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]),
        "moe_combine": (I, [Z, P, P, P, P, P, P, P]),
        "moe_layer_fwd": (I, [Z, ctypes.POINTER(MoeWeights), P, P, ctypes.POINTER(MoeLayerIO), P, S, P]),
        "moe_backward_workspace_bytes": (S, [Z]),
        "moe_transpose_weights": (I, [Z, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeightsT), P]),
        "moe_layer_bwd": (I, [Z, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeightsT), P, P, ctypes.c_float,
                              ctypes.c_float, ctypes.POINTER(MoeLayerIO), ctypes.POINTER(MoeGrads), P, S, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if lib.moe_abi_version() != MOE_ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has struct layout version {lib.moe_abi_version()}, this binding "
                          f"version {MOE_ABI_VERSION}: rebuild the library")
    return lib


_lib = _load()


def config_struct(cfg):
    """moe_config from any object (or dict) carrying the C field names."""
    if isinstance(cfg, dict):
        get = lambda n: cfg[n] if (n in cfg or n not in _OPTIONAL_FIELDS) else 0
    else:
        get = lambda n: getattr(cfg, n) if (hasattr(cfg, n) or n not in _OPTIONAL_FIELDS) else 0
    return MoeConfig(*[int(get(n)) for n in CONFIG_FIELDS])


def _c(cfg):
    return cfg if isinstance(cfg, MoeConfig) else config_struct(cfg)


def _addr(t):
    """Device address of a tensor (None for None); the library reads a dense row-major device buffer."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {tuple(t.stride())} for shape {tuple(t.shape)}")
    return _check_alignment(t.data_ptr())


def _check_alignment(addr):
    """The library moves 16-byte vectors: every device address must be 16-byte aligned."""
    if addr % 16:
        raise ValueError(f"expected a 16-byte aligned device buffer, got address {addr:#x}")
    return addr


def _p(t):
    return None if t is None else ctypes.c_void_p(_addr(t))


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, where):
    if rc != MOE_OK:
        raise MoeError(rc, where)
    return rc


def status_str(status):
    return _lib.moe_status_str(int(status)).decode()


def moe_workspace_bytes(cfg):
    return int(_lib.moe_workspace_bytes(ctypes.byref(_c(cfg))))


def moe_rows_upper_bound(cfg):
    return int(_lib.moe_rows_upper_bound(ctypes.byref(_c(cfg))))


def moe_check_config(cfg):
    return int(_lib.moe_check_config(ctypes.byref(_c(cfg))))


def workspace(cfg, device="cuda"):
    """A uint8 device tensor of moe_workspace_bytes(cfg) bytes (256-byte aligned)."""
    import torch
    n = moe_workspace_bytes(cfg)
    if n == 0:
        raise MoeError(moe_check_config(cfg), "workspace")
    t = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + n]


def _nbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def moe_route(cfg, x, w_router, bias, logits, mode, topk_idx, topk_w, aux_loss, ws, stream=None, sel_bias=None,
              seq_loss=None):
    """moe_route; with a selection bias or a sequence statistic, moe_route_ex."""
    if sel_bias is not None or seq_loss is not None:
        return moe_route_ex(cfg, x, w_router, bias, sel_bias, logits, mode, topk_idx, topk_w, aux_loss, seq_loss, ws,
                            stream)
    c = _c(cfg)
    return _check(_lib.moe_route(ctypes.byref(c), _p(x), _p(w_router), _p(bias), _p(logits), int(mode),
                                 _p(topk_idx), _p(topk_w), _p(aux_loss), _p(ws), _nbytes(ws), _stream(stream)),
                  "moe_route")


def moe_route_ex(cfg, x, w_router, bias, sel_bias, logits, mode, topk_idx, topk_w, aux_loss, seq_loss, ws,
                 stream=None):
    c = _c(cfg)
    return _check(_lib.moe_route_ex(ctypes.byref(c), _p(x), _p(w_router), _p(bias), _p(sel_bias), _p(logits),
                                    int(mode), _p(topk_idx), _p(topk_w), _p(aux_loss), _p(seq_loss), _p(ws),
                                    _nbytes(ws), _stream(stream)), "moe_route_ex")


def moe_sel_bias_update(cfg, load, sel_bias, gamma, stream=None):
    c = _c(cfg)
    return _check(_lib.moe_sel_bias_update(ctypes.byref(c), _p(load), _p(sel_bias), float(gamma), _stream(stream)),
                  "moe_sel_bias_update")


def moe_dispatch(cfg, topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm, ws, stream=None):
    c = _c(cfg)
    return _check(_lib.moe_dispatch(ctypes.byref(c), _p(topk_idx), _p(topk_w), _p(x), _p(demand), _p(counts),
                                    _p(offsets), _p(row_of), _p(src_of), _p(x_perm), _p(ws), _nbytes(ws),
                                    _stream(stream)), "moe_dispatch")


def moe_dispatch_noalloc(cfg, topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm, stream=None):
    c = _c(cfg)
    return _check(_lib.moe_dispatch_noalloc(ctypes.byref(c), _p(topk_idx), _p(topk_w), _p(x), _p(demand), _p(counts),
                                            _p(offsets), _p(row_of), _p(src_of), _p(x_perm), _stream(stream)),
                  "moe_dispatch_noalloc")


def moe_check_topk(cfg, topk_idx, status, stream=None):
    """Checked mode: the count of invalid slots of topk_idx written to status (int32 [1], device)."""
    c = _c(cfg)
    return _check(_lib.moe_check_topk(ctypes.byref(c), _p(topk_idx), _p(status), _stream(stream)), "moe_check_topk")


def moe_expert_ffn(cfg, x_perm, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws,
                   stream=None):
    c = _c(cfg)
    return _check(_lib.moe_expert_ffn(ctypes.byref(c), _p(x_perm), _p(offsets), _p(w1), _p(w3), _p(w2),
                                      _p(y_perm), _p(x_shared), _p(ws1), _p(ws3), _p(ws2), _p(shared_out),
                                      _p(ws), _nbytes(ws), _stream(stream)), "moe_expert_ffn")


def moe_expert_ffn_gather(cfg, x, src_of, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2, shared_out, ws,
                          stream=None):
    c = _c(cfg)
    return _check(_lib.moe_expert_ffn_gather(ctypes.byref(c), _p(x), _p(src_of), _p(offsets), _p(w1), _p(w3),
                                             _p(w2), _p(y_perm), _p(x_shared), _p(ws1), _p(ws3), _p(ws2),
                                             _p(shared_out), _p(ws), _nbytes(ws), _stream(stream)),
                  "moe_expert_ffn_gather")


def moe_combine(cfg, y_perm, row_of, topk_w, residual, shared_out, y, stream=None):
    c = _c(cfg)
    return _check(_lib.moe_combine(ctypes.byref(c), _p(y_perm), _p(row_of), _p(topk_w), _p(residual),
                                   _p(shared_out), _p(y), _stream(stream)), "moe_combine")


def moe_layer_fwd(cfg, weights, x, y, io=None, ws=None, stream=None):
    """weights: dict with moe_weights field names -> tensors (or None).
    io: dict with moe_layer_io field names -> tensors, plus optional 'logits_mode'."""
    c = _c(cfg)
    w = MoeWeights(**{k: _addr(v) for k, v in weights.items()})
    iob = None
    if io is not None:
        kw = {k: _addr(v) for k, v in io.items() if k != "logits_mode"}
        iob = MoeLayerIO(logits_mode=int(io.get("logits_mode", MOE_LOGITS_COMPUTE)), **kw)
    return _check(_lib.moe_layer_fwd(ctypes.byref(c), ctypes.byref(w), _p(x), _p(y),
                                     ctypes.byref(iob) if iob is not None else None, _p(ws), _nbytes(ws),
                                     _stream(stream)), "moe_layer_fwd")


# ---------------------------------------------------------------- backward
def moe_backward_workspace_bytes(cfg):
    return int(_lib.moe_backward_workspace_bytes(ctypes.byref(_c(cfg))))


def backward_workspace(cfg, device="cuda"):
    """A uint8 device tensor of moe_backward_workspace_bytes(cfg) bytes (256-byte aligned)."""
    import torch
    n = moe_backward_workspace_bytes(cfg)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, "backward_workspace")
    t = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + n]


def _weights(weights):
    return MoeWeights(**{k: _addr(v) for k, v in weights.items()})


def moe_transpose_weights(cfg, weights, wt, stream=None):
    """weights: moe_weights field names -> tensors; wt: moe_weights_t field names -> tensors."""
    c = _c(cfg)
    w = _weights(weights)
    t = MoeWeightsT(**{k: _addr(v) for k, v in wt.items()})
    return _check(_lib.moe_transpose_weights(ctypes.byref(c), ctypes.byref(w), ctypes.byref(t), _stream(stream)),
                  "moe_transpose_weights")


def moe_layer_bwd(cfg, weights, wt, x, dy, aux_weight, io, grads, ws, stream=None, seq_weight=0.0):
    """io: the forward's moe_layer_io tensors (dict); grads: moe_grads field names -> tensors."""
    c = _c(cfg)
    w = _weights(weights)
    t = MoeWeightsT(**{k: _addr(v) for k, v in wt.items()})
    kw = {k: _addr(v) for k, v in io.items() if k != "logits_mode"}
    iob = MoeLayerIO(logits_mode=int(io.get("logits_mode", MOE_LOGITS_COMPUTE)), **kw)
    g = MoeGrads(**{k: _addr(v) for k, v in grads.items()})
    return _check(_lib.moe_layer_bwd(ctypes.byref(c), ctypes.byref(w), ctypes.byref(t), _p(x), _p(dy),
                                     float(aux_weight), float(seq_weight), ctypes.byref(iob), ctypes.byref(g),
                                     _p(ws), _nbytes(ws),
                                     _stream(stream)), "moe_layer_bwd")
