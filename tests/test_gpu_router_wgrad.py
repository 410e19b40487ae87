"""Router weight and bias gradients of bf16 layers at float32 accuracy.

In bf16 layers the router weight gradient dW_r = dl^T x runs on bf16 MFMA:
dl (float32) is split into three bf16 planes whose sum is dl to about 2^-24,
and the products with the bf16 x are exact in float32.  So dW_r must match a
float64 evaluation as a float32 computation would, far inside the 2e-2 bar of
the other bf16 gradients.

The one bf16-level input of the router backward is the gate gradient
dg = <dy, F_e(x)>: the layer holds F_e(x) rounded to bf16 (y_perm).  The
reference therefore takes the oracle's softmax, gate-to-probability gradient
and softmax Jacobian in float64, fed with the gate gradients of the GPU's own
y_perm (its bf16 values, exact in float64).  Bar: 1e-6 * max|ref| for dW_r
and dbias.  Its power is checked on the CPU: the oracle's dl rounded to
float32 meets it (the float32 floor), while dl cut to two bf16 planes
(hi + mid) or to one misses it, so a dropped plane, or any bf16 rounding of
dl, fails the GPU test.

The shapes cover the three expert-tile widths (16, 32, 64 experts; 100 experts
per head padded to two 64-expert tiles), two heads (with one and with two
expert tiles per head), renormalised gates, the
affinity keep rule, ragged token counts with several token ranges (the last
one partial, so its final chunk is masked) and head widths of 320 and 576
columns (a partial 256-column tile).
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.moe_backward as OB
import routing_dispatch_expert_router_amd as moe
from moe_inputs import generate, bf16_bits_from_f32
from moe_inputs.configs import MoEConfig
from tests.gpu_util import log, dev, f64
from tests.test_gpu_backward import _forward, _transposed, _grads

BAR = 1e-6
CFGS = [
    MoEConfig("rw_e8_dh320", T=1000, d_model=320, n_heads=1, d_head=320, n_experts=8, top_k=2, d_ff=64, act=1,
              drop=0, act_dtype=1, router_dtype=1, tag=301),
    MoEConfig("rw_h2_e24_renorm", T=777, d_model=256, n_heads=2, d_head=128, n_experts=48, top_k=3, d_ff=64,
              act=1, drop=0, renorm=1, act_dtype=1, router_dtype=0, tag=302),
    MoEConfig("rw_e40_t4133", T=4133, d_model=192, n_heads=1, d_head=192, n_experts=40, top_k=4, d_ff=64, act=0,
              drop=0, act_dtype=1, router_dtype=1, tag=303),
    MoEConfig("rw_e100_dh576_affinity", T=2100, d_model=576, n_heads=1, d_head=576, n_experts=100, top_k=6,
              d_ff=64, act=1, drop=2, keep_num=9, keep_den=10, act_dtype=1, router_dtype=1, tag=304),
    # two heads of 80 experts: each head padded to 128, two 64-expert tiles per head
    MoEConfig("rw_h2_e80", T=1500, d_model=256, n_heads=2, d_head=128, n_experts=160, top_k=2, d_ff=64, act=1,
              drop=0, act_dtype=1, router_dtype=1, tag=305),
]


def _dy(cfg):
    a = np.random.default_rng([5, cfg.tag]).standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    return bf16_bits_from_f32(a)


def _lam(cfg):
    return 0.01 if cfg.n_heads == 1 else 0.0


def _bf16(a):
    """float64 values rounded to float32, then to bf16 (round to nearest even), as float64."""
    return oracle.decode(bf16_bits_from_f32(np.asarray(a, np.float32)))


def _dw_router(cfg, dl, u):
    Eh, dh = cfg.n_experts // cfg.n_heads, cfg.d_head
    w = np.empty((cfg.n_experts, dh))
    for h in range(cfg.n_heads):
        w[h * Eh:(h + 1) * Eh] = dl[:, h * Eh:(h + 1) * Eh].T @ u[:, h * dh:(h + 1) * dh]
    return w


def _reference(cfg, inp, topk_idx, kept):
    P = OB.params_of(inp)
    return P, OB.backward(cfg, P, topk_idx, kept, oracle.decode(_dy(cfg)), _lam(cfg))


@pytest.mark.parametrize("cfg", CFGS[:2], ids=lambda c: c.name)
def test_bar_separates_float32_from_bf16_planes(cfg):
    """CPU: float32 dl meets the bar; dl cut to two bf16 planes, or one, does not."""
    inp = generate(cfg)
    out = oracle.forward(cfg, inp)
    kept = np.ones(cfg.T * cfg.k_total, bool)
    P, ref = _reference(cfg, inp, out["topk_idx"], kept)
    sc = np.max(np.abs(ref["dw_router"]))
    rel = lambda d: np.max(np.abs(_dw_router(cfg, d, P["x"]) - ref["dw_router"])) / sc
    d32 = ref["dl"].astype(np.float32).astype(np.float64)
    hi = _bf16(d32)
    mid = _bf16(d32 - hi)
    assert rel(d32) < 0.1 * BAR
    assert rel(hi + mid) > 2 * BAR
    assert rel(hi) > 100 * BAR


def _reference_from_gpu_outputs(cfg, P, io, dy64, lam):
    """dW_r and dbias (float64) from the gate gradients of the GPU's own expert outputs y_perm."""
    T, K, H, dh = cfg.T, cfg.k_total, cfg.n_heads, cfg.d_head
    k = K // H
    idx = io["topk_idx"].cpu().numpy().astype(np.int64)
    row_of = io["row_of"].cpu().numpy()
    kept = row_of >= 0
    yp = f64(io["y_perm"])
    dyh = dy64.reshape(T, H, dh)[:, np.arange(K) // k, :]  # [T, K, dh]: each slot's head slice of dy
    dg = np.where(kept, np.einsum("tkc,tkc->tk", dyh, yp[np.maximum(row_of, 0)]), 0.0)
    u = P["x"]
    p = OB._probs(cfg, P, u)
    g, S = OB._gate_values(cfg, P, np.take_along_axis(p, idx, axis=1), idx)
    dp = np.zeros_like(p)
    np.add.at(dp, (np.arange(T)[:, None].repeat(K, 1), idx), OB._gate_to_prob_grad(cfg, g, S, dg))
    if lam:
        dp += lam * np.bincount(idx.reshape(-1), minlength=cfg.n_experts)[None, :] / (T * T)
    dl = OB._head_softmax_backward(cfg, p, dp)
    return dict(dw_router=_dw_router(cfg, dl, u), dbias=dl.sum(axis=0))


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_router_gradients_float32_accurate(cfg):
    log(f"router gradients {cfg.name}")
    inp = generate(cfg)
    out = oracle.forward(cfg, inp)
    W, x, io = _forward(cfg, inp, out["logits"])
    assert np.array_equal(io["topk_idx"].cpu().numpy(), out["topk_idx"])
    G = _grads(cfg)
    dy_h = _dy(cfg)
    moe.moe_layer_bwd(cfg, W, _transposed(cfg, W), x, dev(dy_h), _lam(cfg), io, G, moe.backward_workspace(cfg))
    torch.cuda.synchronize()
    ref = _reference_from_gpu_outputs(cfg, OB.params_of(inp), io, oracle.decode(dy_h), _lam(cfg))
    for name in ("dw_router", "dbias"):
        got, want = f64(G[name]), ref[name]
        sc = np.max(np.abs(want))
        err = np.max(np.abs(got - want))
        log(f"  {name:9s} max|ref| {sc:.3g}  rel err {err / sc:.3g}")
        assert err <= BAR * sc, name
