"""GPU parity of the layer backward (moe_layer_bwd) against the float64 backward oracle.

One-head layers, several routing heads with and without the latent projections.
The forward runs on the GPU with the oracle's float32 scores loaded (routing
identical); the oracle backward then takes the GPU's own keep decisions, so
both sides differentiate the same function.  Bars: every gradient within
2e-2 * max|ref| (bf16 layers) or 1e-4 * max|ref| (float32 layers); two
backward runs bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.moe_backward as OB
import routing_dispatch_expert_router_amd as moe
from moe_inputs import SMALL, MoEConfig, generate, bf16_bits_from_f32
from tests.gpu_util import log, dev, f64, empty_act, i32, f32, tol, weights_dev

pytestmark = pytest.mark.gpu

ONE_HEAD = [c for c in SMALL if c.n_heads == 1 and not c.latent_proj]
MULTI_HEAD = [c for c in SMALL if c.n_heads > 1]
EDGE = [
    MoEConfig("bwd_edge_relu_bf16", T=70, d_model=128, n_heads=1, d_head=128, n_experts=5, top_k=2, d_ff=192,
              act=0, drop=1, capacity=20, n_shared=1, tag=70),
    MoEConfig("bwd_edge_k1_noresid", T=33, d_model=64, n_heads=1, d_head=64, n_experts=3, top_k=1, d_ff=64,
              residual=0, renorm=1, tag=71),
    # two heads without projections (d_model = 2 * d_head), renormalised top-2 per head, ragged T
    MoEConfig("bwd_edge_two_heads", T=45, d_model=256, n_heads=2, d_head=128, n_experts=10, top_k=2, d_ff=128,
              renorm=1, drop=1, capacity=12, tag=72),
    # few output tiles per weight gradient and many tokens: the K-split paths (per expert and shared)
    MoEConfig("bwd_edge_splitk", T=2048, d_model=256, n_heads=1, d_head=256, n_experts=4, top_k=2, d_ff=128,
              n_shared=1, renorm=1, tag=74),
    # latent heads with a d_head that is not a multiple of 256, float32
    MoEConfig("bwd_edge_latent_f32", T=29, d_model=128, n_heads=3, d_head=64, n_experts=12, top_k=1, d_ff=64,
              latent_proj=1, act=0, act_dtype=0, router_dtype=0, tag=73),
]
CFGS = ONE_HEAD + MULTI_HEAD + EDGE
IDS = [c.name for c in CFGS]
LAM = 0.5


def _lam(cfg):
    """The aux loss exists for one routing head only."""
    return LAM if cfg.n_heads == 1 else 0.0


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _forward(cfg, inp, logits, gu=False, want_y=False):
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = moe.moe_rows_upper_bound(cfg)
    io = dict(logits=dev(logits), logits_mode=moe.MOE_LOGITS_LOAD, topk_idx=i32(T, K), topk_w=f32(T, K),
              demand=i32(E), counts=i32(E), offsets=i32(E + 1), row_of=i32(T, K), src_of=i32(max(Rm, 1)),
              y_perm=empty_act(cfg, max(Rm, 1), cfg.d_head),
              z=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None,
              o=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None)
    if gu:  # the routed pre-activations, kept for the backward
        io["gu"] = empty_act(cfg, max(Rm, 1), (2 if cfg.act == 1 else 1) * cfg.d_ff)
    W = weights_dev(cfg, inp)
    x = dev(inp.x)
    y = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, W, x, y, io, moe.workspace(cfg))
    torch.cuda.synchronize()
    return (W, x, io, y) if want_y else (W, x, io)


def _transposed(cfg, W):
    m = 2 if cfg.act == 1 else 1
    adt = torch.bfloat16 if cfg.act_dtype == 1 else torch.float32
    E, dh, F, d = cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
    fs = cfg.n_shared * F
    D = cfg.d_latent
    wt = dict(w13t=torch.empty(E, dh, m * F, dtype=adt, device="cuda"),
              w2t=torch.empty(E, F, dh, dtype=adt, device="cuda"),
              ws13t=torch.empty(d, m * fs, dtype=adt, device="cuda") if fs else None,
              ws2t=torch.empty(fs, d, dtype=adt, device="cuda") if fs else None,
              w_in_t=torch.empty(d, D, dtype=adt, device="cuda") if cfg.latent_proj else None,
              w_out_t=torch.empty(D, d, dtype=adt, device="cuda") if cfg.latent_proj else None)
    moe.moe_transpose_weights(cfg, W, wt)
    return wt


def _grads(cfg):
    adt = torch.bfloat16 if cfg.act_dtype == 1 else torch.float32
    E, dh, F, d = cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
    fs = cfg.n_shared * F
    z = lambda *s: torch.full(s, float("nan"), dtype=adt, device="cuda")
    D = cfg.d_latent
    return dict(dx=z(cfg.T, d), dw_router=f32(E, dh), dbias=f32(E), dw1=z(E, F, dh),
                dw3=z(E, F, dh) if cfg.act == 1 else None, dw2=z(E, dh, F),
                dws1=z(fs, d) if fs else None, dws3=z(fs, d) if (fs and cfg.act == 1) else None,
                dws2=z(d, fs) if fs else None,
                dw_in=z(D, d) if cfg.latent_proj else None, dw_out=z(d, D) if cfg.latent_proj else None)


def _dy(cfg):
    rng = np.random.default_rng([99, cfg.tag])
    a = rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    return bf16_bits_from_f32(a) if cfg.act_dtype == 1 else a


def _inputs(cfg):
    return generate(cfg)


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_backward_matches_oracle(cfg):
    log(f"backward {cfg.name}")
    inp = _inputs(cfg)
    out = oracle.forward(cfg, inp)
    W, x, io = _forward(cfg, inp, out["logits"])
    assert np.array_equal(io["topk_idx"].cpu().numpy(), out["topk_idx"])
    wt = _transposed(cfg, W)
    dy_h = _dy(cfg)
    dy = dev(dy_h)
    G = _grads(cfg)
    ws = moe.backward_workspace(cfg)
    lam = _lam(cfg)
    moe.moe_layer_bwd(cfg, W, wt, x, dy, lam, io, G, ws)
    torch.cuda.synchronize()
    # the oracle differentiates the same decisions: the GPU's top-k and keep mask
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    P = OB.params_of(inp)
    # (with latent_proj the GPU's experts read its own stored z, the oracle float64 z: a rounding the bars cover)
    ref = OB.backward(cfg, P, io["topk_idx"].cpu().numpy(), kept, oracle.decode(dy_h), lam)
    pairs = [("dx", "dx"), ("dw_router", "dw_router"), ("dbias", "dbias"), ("dw1", "dw1"), ("dw2", "dw2")]
    if cfg.act == 1:
        pairs.append(("dw3", "dw3"))
    if cfg.n_shared:
        pairs += [("dws1", "dws1"), ("dws2", "dws2")] + ([("dws3", "dws3")] if cfg.act == 1 else [])
    if cfg.latent_proj:
        pairs += [("dw_in", "dw_in"), ("dw_out", "dw_out")]
    for gk, rk in pairs:
        got, want = f64(G[gk]), ref[rk]
        scale = max(np.max(np.abs(want)), 1e-30)
        err = np.max(np.abs(got - want))
        log(f"  {gk:10s} max|ref| {scale:.3g}  rel err {err / scale:.3g}")
        assert np.all(np.isfinite(got)), gk
        assert err <= tol(cfg) * scale, gk


@pytest.mark.parametrize("cfg", [ONE_HEAD[1], EDGE[0], MULTI_HEAD[0]], ids=lambda c: c.name)
def test_backward_deterministic(cfg):
    inp = _inputs(cfg)
    out = oracle.forward(cfg, inp)
    W, x, io = _forward(cfg, inp, out["logits"])
    wt = _transposed(cfg, W)
    dy = dev(_dy(cfg))
    ws = moe.backward_workspace(cfg)
    G1, G2 = _grads(cfg), _grads(cfg)
    moe.moe_layer_bwd(cfg, W, wt, x, dy, _lam(cfg), io, G1, ws)
    moe.moe_layer_bwd(cfg, W, wt, x, dy, _lam(cfg), io, G2, ws)
    torch.cuda.synchronize()
    for k in G1:
        if G1[k] is not None:
            assert torch.equal(_bits(G1[k]), _bits(G2[k])), k


def test_backward_rejects_aux_with_several_heads():
    """The aux loss is defined for one head: a nonzero weight with several heads is refused before launching."""
    cfg = SMALL[4]
    inp = _inputs(cfg)
    out = oracle.forward(cfg, inp)
    W, x, io = _forward(cfg, inp, out["logits"])
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_bwd(cfg, W, _transposed(cfg, W), x, dev(_dy(cfg)), 0.5, io, _grads(cfg),
                          moe.backward_workspace(cfg))
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED


def _grouped(cfg):
    """The routed experts run the grouped GEMM (not the fused narrow-expert MLP): the layers
    whose forward keeps the pre-activations for the backward."""
    return cfg.act_dtype == 0 or cfg.d_head not in (64, 128, 256)


GU_CFGS = [c for c in CFGS if _grouped(c)] + [
    # bf16 ReLU experts on the grouped GEMM (d_head 192)
    MoEConfig("bwd_gu_relu_bf16", T=70, d_model=192, n_heads=1, d_head=192, n_experts=5, top_k=2, d_ff=128,
              act=0, drop=1, capacity=20, tag=75),
    # experts of about 1024 rows: 256-row tiles and their tails keep the pre-activations too
    MoEConfig("bwd_gu_tall", T=2048, d_model=320, n_heads=1, d_head=320, n_experts=4, top_k=2, d_ff=128,
              renorm=1, tag=76),
]


@pytest.mark.parametrize("cfg", GU_CFGS, ids=lambda c: c.name)
def test_backward_with_kept_preactivations(cfg):
    """moe_layer_fwd keeps the routed pre-activations in io.gu; moe_layer_bwd then reads them
    instead of recomputing the gate/up products.  The forward's output is bitwise the same,
    and every gradient meets the same bars against the backward oracle."""
    log(f"backward with kept pre-activations {cfg.name}")
    inp = _inputs(cfg)
    out = oracle.forward(cfg, inp)
    W, x, io0, y0 = _forward(cfg, inp, out["logits"], want_y=True)
    _, _, io, y1 = _forward(cfg, inp, out["logits"], gu=True, want_y=True)
    assert torch.equal(_bits(y0), _bits(y1))
    wt = _transposed(cfg, W)
    dy_h = _dy(cfg)
    G = _grads(cfg)
    lam = _lam(cfg)
    moe.moe_layer_bwd(cfg, W, wt, x, dev(dy_h), lam, io, G, moe.backward_workspace(cfg))
    torch.cuda.synchronize()
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    ref = OB.backward(cfg, OB.params_of(inp), io["topk_idx"].cpu().numpy(), kept, oracle.decode(dy_h), lam)
    names = ["dx", "dw_router", "dbias", "dw1", "dw2"] + (["dw3"] if cfg.act == 1 else [])
    if cfg.n_shared:
        names += ["dws1", "dws2"] + (["dws3"] if cfg.act == 1 else [])
    if cfg.latent_proj:
        names += ["dw_in", "dw_out"]
    for k in names:
        got, want = f64(G[k]), ref[k]
        scale = max(np.max(np.abs(want)), 1e-30)
        err = np.max(np.abs(got - want))
        log(f"  {k:10s} max|ref| {scale:.3g}  rel err {err / scale:.3g}")
        assert np.all(np.isfinite(got)), k
        assert err <= tol(cfg) * scale, k
