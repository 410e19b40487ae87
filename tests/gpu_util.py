"""Helpers for the GPU parity tests: host arrays <-> device tensors, oracle runs."""
import functools
import sys

import numpy as np
import torch

import oracle
from moe_inputs import generate, bf16_bits_from_f32


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    """numpy host array (uint16 = bf16 bits) -> device tensor."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def f64(t):
    """device tensor -> float64 numpy (bf16 decoded exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def act_round(cfg, a64):
    """Round float64 values to the layer's activation storage (bf16 bits or float32)."""
    if cfg.act_dtype == 1:
        return bf16_bits_from_f32(np.asarray(a64, np.float32))
    return np.asarray(a64, np.float32)


def empty_act(cfg, *shape):
    return torch.empty(*shape, dtype=torch.bfloat16 if cfg.act_dtype == 1 else torch.float32, device="cuda")


def i32(*shape):
    return torch.full(shape, -7, dtype=torch.int32, device="cuda")


def f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


@functools.lru_cache(maxsize=8)
def cached_inputs(cfg):
    return generate(cfg)


def tol(cfg):
    """max-abs-error bound relative to max|ref|: 1e-4 for float32 layers, 2e-2 for bf16."""
    return 1e-4 if cfg.act_dtype == 0 else 2e-2


def weights_dev(cfg, inp):
    return dict(w_router=dev(inp.w_router), router_bias=dev(inp.bias), w1=dev(inp.w1), w3=dev(inp.w3),
                w2=dev(inp.w2), ws1=dev(inp.ws1), ws3=dev(inp.ws3), ws2=dev(inp.ws2), w_in=dev(inp.w_in),
                w_out=dev(inp.w_out), sel_bias=dev(getattr(inp, "sel_bias", None)))


def routing_margin(cfg, l32):
    """Per token, the smallest gap between a chosen and an unchosen score (per head), on the oracle's scores."""
    T, H, Eh, k = cfg.T, cfg.n_heads, cfg.e_per_head, cfg.top_k
    gap = np.full(T, np.inf)
    for h in range(H):
        s = np.sort(l32[:, h * Eh:(h + 1) * Eh].astype(np.float64), axis=1)[:, ::-1]
        if k < Eh:
            gap = np.minimum(gap, s[:, k - 1] - s[:, k])
        if k > 1:
            gap = np.minimum(gap, np.min(s[:, :k - 1] - s[:, 1:k], axis=1))
        if cfg.n_groups:
            g = np.sort(l32[:, h * Eh:(h + 1) * Eh].astype(np.float64).reshape(T, cfg.n_groups, -1).max(axis=2),
                        axis=1)[:, ::-1]
            if cfg.topk_groups < cfg.n_groups:
                gap = np.minimum(gap, g[:, cfg.topk_groups - 1] - g[:, cfg.topk_groups])
    return gap
