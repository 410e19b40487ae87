"""Plant one plausible mistake at a time into the CPU oracle; the pins must catch each.

Every mutant replaces one oracle function for the duration of the test
(monkeypatch, on the CPU); the pin suite from oracle_pins must then fail.
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
from tests import oracle_pins as P

_orig = {n: getattr(O, n) for n in ("router_logits", "select_topk", "softmax", "gates", "aux_loss", "keep_capacity",
                                     "keep_affinity", "permutation", "expert_ffn", "silu", "forward",
                                     "route")}


def m_logits_no_bias(xr, w_r, bias=None):
    return _orig["router_logits"](xr, w_r, None)


def m_logits_bias_twice(xr, w_r, bias=None):
    return _orig["router_logits"](xr, w_r, None if bias is None else 2 * np.asarray(bias, np.float64))


def m_logits_transposed(xr, w_r, bias=None):
    # the head's weight block used transposed (it is square in the hand example)
    w = w_r.T if w_r.shape[0] == w_r.shape[1] else w_r
    return _orig["router_logits"](xr, w, bias)


def m_ties_high(l32, k, n_groups=0, topk_groups=0):
    l32 = np.asarray(l32, np.float32)[:, ::-1]
    E = l32.shape[1]
    return (E - 1 - _orig["select_topk"](l32, k, 0, 0)).astype(np.int32)


def m_group_sum(l32, k, n_groups=0, topk_groups=0):
    if not n_groups:
        return _orig["select_topk"](l32, k)
    l32 = np.asarray(l32, np.float32)
    T, E = l32.shape
    gsz = E // n_groups
    gs = l32.reshape(T, n_groups, gsz).sum(axis=2)
    gsel = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
    allow = np.zeros((T, n_groups), bool)
    allow[np.arange(T)[:, None], gsel] = True
    l2 = np.where(np.repeat(allow, gsz, axis=1), l32, np.float32(-np.inf))
    return np.argsort(-l2, axis=1, kind="stable")[:, :k].astype(np.int32)


def m_softmax_noexp(l):
    l = np.asarray(l, np.float64)
    e = l - l.min(axis=-1, keepdims=True) + 1.0
    return e / e.sum(axis=-1, keepdims=True)


def m_no_renorm(p, idx, renorm):
    return _orig["gates"](p, idx, 0)


def m_aux_top1(p, idx):
    return _orig["aux_loss"](p, idx[:, :1])


def m_cap_le(e_flat, n_experts, C):
    return _orig["keep_capacity"](e_flat, n_experts, C + 1)


def m_aff_floor(e_flat, w32, n_experts, num, den):
    kept = np.zeros(len(e_flat), bool)
    for e in range(n_experts):
        mem = np.nonzero(e_flat == e)[0].tolist()
        keep = num * len(mem) // den
        kept[sorted(mem, key=lambda a: (-float(w32[a]), a))[:keep]] = True
    return kept


def m_aff_ties_high(e_flat, w32, n_experts, num, den):
    kept = np.zeros(len(e_flat), bool)
    for e in range(n_experts):
        mem = np.nonzero(e_flat == e)[0].tolist()
        keep = (num * len(mem) + den - 1) // den
        kept[sorted(mem, key=lambda a: (-float(w32[a]), -a))[:keep]] = True
    return kept


def m_perm_desc(e_flat, kept, n_experts):
    demand, counts, offsets, row_of, src_of = _orig["permutation"](e_flat, kept, n_experts)
    src2 = src_of.copy()
    for e in range(n_experts):
        src2[offsets[e]:offsets[e + 1]] = src_of[offsets[e]:offsets[e + 1]][::-1]
    row2 = row_of.copy()
    row2[src2] = np.arange(len(src2))
    return demand, counts, offsets, row2, src2


def m_ffn_swap(v, w1, w3, w2, act):
    if act == 0:
        return _orig["expert_ffn"](v, w1, w3, w2, act)
    return _orig["expert_ffn"](v, w3, w1, w2, act)


def m_silu_sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def m_ffn_relu_shift(v, w1, w3, w2, act):
    if act == 1:
        return _orig["expert_ffn"](v, w1, w3, w2, act)
    return (np.maximum(v @ w1.T, 0.0) + 1e-3) @ w2.T


def _wrap_forward(mod):
    def f(cfg, inp, logits=None, tokens=None, want_xperm=False):
        out = _orig["forward"](cfg, inp, logits, tokens, want_xperm)
        return mod(cfg, inp, out)
    return f


def _no_residual(cfg, inp, out):
    if cfg.residual and not cfg.latent_proj:
        out["y"] = out["y"] - O.decode(inp.x)[out["tokens"]]
    return out


def _ungated(cfg, inp, out):
    # recompute the routed sum with unit gates
    w = out["topk_w"]
    out2 = dict(out)
    saved = O.gates
    try:
        O.gates = lambda p, idx, renorm: np.ones(idx.shape)
        out2 = _orig["forward"](cfg, inp, None, out["tokens"], "x_perm" in out)
    finally:
        O.gates = saved
    out2["topk_w"] = w
    return out2


def m_route_head0(cfg, zr, w_router, bias=None, logits=None, sel_bias=None):
    if cfg.n_heads == 1 or zr is None:
        return _orig["route"](cfg, zr, w_router, bias, logits, sel_bias)
    z0 = np.tile(zr[:, :cfg.d_head], (1, cfg.n_heads))
    return _orig["route"](cfg, z0, w_router, bias, logits, sel_bias)


MUTANTS = [
    ("router_logits", m_logits_no_bias), ("router_logits", m_logits_bias_twice),
    ("router_logits", m_logits_transposed),
    ("select_topk", m_ties_high), ("select_topk", m_group_sum), ("softmax", m_softmax_noexp),
    ("gates", m_no_renorm), ("aux_loss", m_aux_top1), ("keep_capacity", m_cap_le),
    ("keep_affinity", m_aff_floor), ("keep_affinity", m_aff_ties_high),
    ("permutation", m_perm_desc), ("expert_ffn", m_ffn_swap), ("silu", m_silu_sigmoid),
    ("expert_ffn", m_ffn_relu_shift), ("forward", _wrap_forward(_no_residual)),
    ("forward", _wrap_forward(_ungated)), ("route", m_route_head0),
]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=lambda v: getattr(v, "__name__", str(v)))
def test_pins_catch_mutant(name, mut, monkeypatch):
    monkeypatch.setattr(O, name, mut)
    caught = []
    for check in P.ALL:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {mut.__name__} in {name}"
