"""Seeded generator for the MoE layer's inputs and weights (recipe in the package docstring)."""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import MoEConfig, BF16

# tensor tags: one independent stream per tensor (and per expert slice)
_TAG = {"x": 1, "w_in": 2, "w_router": 3, "w1": 4, "w3": 5, "w2": 6,
        "ws1": 7, "ws3": 8, "ws2": 9, "w_out": 10}


def bf16_bits_from_f32(a):
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Inputs:
    cfg: MoEConfig
    x: np.ndarray                       # [T, d_model]
    w_router: np.ndarray                # [E, d_head]  (== [H, E_h, d_head])
    bias: np.ndarray = None             # [E] float32 or None
    w1: np.ndarray = None               # [E, d_ff, d_head]
    w3: np.ndarray = None               # [E, d_ff, d_head] (SwiGLU only)
    w2: np.ndarray = None               # [E, d_head, d_ff]
    ws1: np.ndarray = None              # [n_s*d_ff, d_model]
    ws3: np.ndarray = None
    ws2: np.ndarray = None              # [d_model, n_s*d_ff]
    w_in: np.ndarray = None             # [H*d_head, d_model]
    w_out: np.ndarray = None            # [d_model, H*d_head]
    sel_bias: np.ndarray = None         # [E] float32 or None: selection-only expert bias
    meta: dict = field(default_factory=dict)

    def is_bf16(self, name):
        a = getattr(self, name)
        return a is not None and a.dtype == np.uint16


def _fill(out, cfg, name, index, scale, bf16):
    """Fill `out` (a view) with N(0, scale^2) from the stream (seed, tag, tensor, index)."""
    rng = np.random.default_rng([cfg.seed, cfg.tag, _TAG[name], index])
    a = rng.standard_normal(out.size, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    a = a.reshape(out.shape)
    if bf16:
        out[...] = bf16_bits_from_f32(a)
    else:
        out[...] = a


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(cfg: MoEConfig, threads=None) -> Inputs:
    """Draw every input of `cfg` (host arrays)."""
    bf = cfg.act_dtype == BF16
    adt = np.uint16 if bf else np.float32
    rdt = np.uint16 if cfg.router_dtype == BF16 else np.float32
    T, d, H, dh, E, dff = cfg.T, cfg.d_model, cfg.n_heads, cfg.d_head, cfg.n_experts, cfg.d_ff
    dl = H * dh
    jobs = []
    x = np.empty((T, d), adt)
    # x in row blocks so large activations also generate in parallel
    rb = max(1, (1 << 22) // max(d, 1))
    for i, r0 in enumerate(range(0, T, rb)):
        jobs.append((x[r0:r0 + rb], "x", i, 1.0, bf))
    w_in = w_out = None
    if cfg.latent_proj:
        w_in = np.empty((dl, d), adt)
        jobs.append((w_in, "w_in", 0, 1.0 / np.sqrt(d), bf))
        w_out = np.empty((d, dl), adt)
        jobs.append((w_out, "w_out", 0, 1.0 / np.sqrt(dl), bf))
    w_router = np.empty((E, dh), rdt)
    jobs.append((w_router, "w_router", 0, 1.0 / np.sqrt(dh), rdt == np.uint16))
    w1 = np.empty((E, dff, dh), adt)
    w2 = np.empty((E, dh, dff), adt)
    w3 = np.empty((E, dff, dh), adt) if cfg.act == 1 else None
    for e in range(E):
        jobs.append((w1[e], "w1", e, 1.0 / np.sqrt(dh), bf))
        if w3 is not None:
            jobs.append((w3[e], "w3", e, 1.0 / np.sqrt(dh), bf))
        jobs.append((w2[e], "w2", e, 1.0 / np.sqrt(dff), bf))
    ws1 = ws3 = ws2 = None
    if cfg.n_shared:
        fs = cfg.n_shared * dff
        ws1 = np.empty((fs, d), adt)
        jobs.append((ws1, "ws1", 0, 1.0 / np.sqrt(d), bf))
        if cfg.act == 1:
            ws3 = np.empty((fs, d), adt)
            jobs.append((ws3, "ws3", 0, 1.0 / np.sqrt(d), bf))
        ws2 = np.empty((d, fs), adt)
        jobs.append((ws2, "ws2", 0, 1.0 / np.sqrt(dff), bf))
    n = threads or _threads()
    if n == 1:
        for j in jobs:
            _fill(j[0], cfg, *j[1:])
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(lambda j: _fill(j[0], cfg, *j[1:]), jobs))
    bias = None
    if cfg.zipf_s > 0:
        eh = E // H
        b = (-cfg.zipf_s * np.log(np.arange(1, eh + 1, dtype=np.float64))).astype(np.float32)
        bias = np.tile(b, H)
    sel_bias = None
    if cfg.sel_bias_steps > 0:
        # a balancing bias as it stands after some +-0.001 updates
        rng = np.random.default_rng([cfg.seed, cfg.tag, 11, 0])
        n = rng.integers(-cfg.sel_bias_steps, cfg.sel_bias_steps + 1, size=E)
        sel_bias = (n * 0.001).astype(np.float32)
    return Inputs(cfg=cfg, x=x, w_router=w_router, bias=bias, w1=w1, w3=w3, w2=w2,
                  ws1=ws1, ws3=ws3, ws2=ws2, w_in=w_in, w_out=w_out, sel_bias=sel_bias)
