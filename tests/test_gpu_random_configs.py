"""Seeded random layer configurations: forward and backward through the C ABI against the oracle.

Each case draws a small layer (routing heads with or without the latent
projections, group-limited selection, a keep rule, expert choice, a
selection bias in or out of the gate, the per-sequence statistic, shared
experts, ReLU or SwiGLU, float32 or bf16, a ragged token count) and its
seeded inputs, then runs moe_layer_fwd with the oracle's float32 scores
loaded and checks:
  * the choices equal the oracle's (with a selection bias the GPU forms the
    keys p + b from its own exp: a token may differ only at an oracle key
    near-tie);
  * the keep rule: the oracle's rule on the GPU's own choices and gates
    gives exactly the GPU's counts, offsets and permutation, and (choices
    equal) a keep decision differs from the oracle's only at a gate near-tie;
  * y against the oracle's y for the GPU's own decisions (top-k and keep
    mask), within 2e-2 (bf16) or 1e-4 (float32) of max|y|;
  * the per-sequence statistic within 1e-5 relative;
  * every gradient of moe_layer_bwd against the backward oracle for those
    decisions, within the same bars (the bias gradient, a sum over tokens, against
    the larger of its own size and its terms' root sum of squares); for ReLU layers plus, element by element,
    the terms of the pre-activations the oracle finds within float32 (and,
    with the latent projections, the stored latent's) reach of 0, whose
    mask the GPU may decide the other way.
moe_route also runs on each case computing its own scores (the router
product's shape variants): scores within 1e-5 of max|l|, choices equal up to
near-ties, gates within 1e-5.
The draws are fixed (seed per case), so a failure names a reproducible case.
Besides the small draws: larger layers (300-3000 tokens, widths up to 512: several
row and column tiles per expert), larger layers of the routing variants, and small
and large layers whose forward keeps the pre-activations for the backward; a few of
each by default, N of each with the environment variable MOE_RANDOM_SWEEP=N (swept
at N = 150-200 on MI355X).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.moe_backward as OB
import routing_dispatch_expert_router_amd as moe
from moe_inputs import generate, bf16_bits_from_f32
from moe_inputs.configs import MoEConfig
from tests.gpu_util import (log, dev, f64, empty_act, i32, f32, tol, weights_dev, routing_margin, check_keep,
                            relu_tie_allowance, act_round)
from tests.test_gpu_backward import _transposed, _grads

N_CASES = 24


def draw(i):
    """The i-th random configuration (always a valid, supported one)."""
    rng = np.random.default_rng([2024, i])
    H = int(rng.choice([1, 1, 1, 2, 4]))
    latent = int((H > 1 and rng.random() < 0.6) or (H == 1 and rng.random() < 0.15))
    dh = int(rng.choice([64, 128, 192]))
    d_model = H * dh if not latent else int(rng.choice([64, 128, 256]))
    Eh = int(rng.integers(1, 25))
    ec = H == 1 and not latent and rng.random() < 0.2
    top_k = 1 if ec else int(rng.integers(1, min(Eh, 8) + 1))
    n_groups = topk_groups = 0
    if not ec:
        divs = [g for g in (2, 3, 4) if Eh % g == 0 and Eh // g >= 1]
        if divs and rng.random() < 0.35:
            n_groups = int(rng.choice(divs))
            need = -(-top_k // (Eh // n_groups))  # groups needed to hold top_k experts
            topk_groups = int(rng.integers(need, n_groups + 1))
    renorm = 0 if ec else int(rng.integers(0, 2))
    seq_len, T = 0, int(rng.integers(1, 261))
    if H == 1 and rng.random() < 0.3:
        seq_len = int(rng.integers(1, 65))
        T = seq_len * int(rng.integers(1, 5))
    if ec:
        drop, capacity = 1, int(rng.integers(0, T + 5))
    else:
        drop = int(rng.integers(0, 3))
        capacity = int(rng.integers(0, -(-T * top_k // Eh) * 2 + 2)) if drop == 1 else 0
    keep_den = int(rng.integers(1, 11))
    keep_num = int(rng.integers(1, keep_den + 1))
    f32_layer = rng.random() < 0.25
    act_dtype = 0 if f32_layer else 1
    router_dtype = 0 if f32_layer else int(rng.integers(0, 2))
    sel_steps = sel_gate = 0
    if not ec and rng.random() < 0.3:
        sel_steps = 5
        sel_gate = 0 if renorm else int(rng.integers(0, 2))  # the backward refuses a bias inside renormalised gates
    cfg = MoEConfig(
        f"rand{i:02d}", T=T, d_model=d_model, n_heads=H, d_head=dh, n_experts=H * Eh, top_k=top_k,
        n_groups=n_groups, topk_groups=topk_groups, renorm=renorm, drop=drop, capacity=capacity,
        keep_num=keep_num, keep_den=keep_den, d_ff=int(rng.choice([64, 128, 192])), act=int(rng.integers(0, 2)),
        n_shared=int(rng.integers(0, 3)) if (H == 1 and not latent) else 0, latent_proj=latent,
        residual=int(rng.integers(0, 2)), act_dtype=act_dtype, router_dtype=router_dtype,
        route_mode=1 if ec else 0, sel_bias_gate=sel_gate, seq_len=seq_len,
        zipf_s=float(rng.choice([0.0, 0.0, 1.0])), sel_bias_steps=sel_steps, tag=200 + i)
    return cfg


# plus draws of ReLU layers with the latent projections (bf16 and float32; top-1 per
# head with its folded combine among them), whose mask near-ties the check allows for
CASES = [draw(i) for i in range(N_CASES)] + [draw(i) for i in (76, 85, 125, 166)] + [
    # two experts, both chosen, renormalised: the bias gradient sums 1001 tokens' terms of
    # random sign down to 0.6 % of their magnitudes
    MoEConfig("rand_e2_all", T=1001, d_model=512, n_heads=1, d_head=512, n_experts=2, top_k=2, renorm=1, drop=0,
              keep_num=6, keep_den=10, d_ff=64, act=0, residual=0, act_dtype=1, router_dtype=1, zipf_s=1.0,
              tag=5055)]


def test_draws_are_valid_and_varied():
    """Host-side: every draw is a supported configuration, and the draws cover the options."""
    for c in CASES + LARGE + VARIANT:
        assert moe.moe_check_config(c) == moe.MOE_OK, c
        assert moe.moe_backward_workspace_bytes(c) > 0, c
    assert {c.n_heads for c in CASES} >= {1, 2}
    assert any(c.latent_proj for c in CASES) and any(c.route_mode for c in CASES)
    assert {c.drop for c in CASES} == {0, 1, 2}
    assert any(c.n_groups for c in CASES) and any(c.sel_bias_steps for c in CASES) and any(c.seq_len for c in CASES)
    assert {c.act_dtype for c in CASES} == {0, 1} and {c.act for c in CASES} == {0, 1}


def draw_large(i):
    """The i-th random layer of 300-3000 tokens and widths up to 512 (several row and
    column tiles per expert: the 256-row tiles, their tails and the mixed launches)."""
    rng = np.random.default_rng([4048, i])
    H = int(rng.choice([1, 1, 2, 4]))
    latent = int(H > 1 and rng.random() < 0.6)
    dh = int(rng.choice([64, 128, 192, 256, 320, 512]))
    d_model = H * dh if not latent else int(rng.choice([128, 256, 512]))
    Eh = int(rng.integers(1, 17))
    top_k = int(rng.integers(1, min(Eh, 8) + 1))
    T = int(rng.integers(300, 3001))
    drop = int(rng.integers(0, 3))
    capacity = int(rng.integers(0, -(-T * top_k // Eh) * 2 + 2)) if drop == 1 else 0
    f32_layer = rng.random() < 0.15
    return MoEConfig(f"large{i:03d}", T=T, d_model=d_model, n_heads=H, d_head=dh, n_experts=H * Eh, top_k=top_k,
                     renorm=int(rng.integers(0, 2)), drop=drop, capacity=capacity, keep_num=int(rng.integers(5, 11)),
                     keep_den=10, d_ff=int(rng.choice([64, 128, 256, 512])), act=int(rng.integers(0, 2)),
                     n_shared=int(rng.integers(0, 2)) if (H == 1 and not latent) else 0, latent_proj=latent,
                     residual=int(rng.integers(0, 2)), act_dtype=0 if f32_layer else 1,
                     router_dtype=0 if f32_layer else int(rng.integers(0, 2)),
                     zipf_s=float(rng.choice([0.0, 1.0, 1.2])), tag=5000 + i)


def draw_variant(i):
    """The i-th random layer of 300-2500 tokens in one of five routing families:
    group-limited with the affinity keep and shared experts, expert choice, the
    balancing bias with the per-sequence statistic, multi-head latent top-1 per head
    (the fused MLP's folded combine), multi-head latent with any k and keep rule."""
    rng = np.random.default_rng([6060, i])
    kind = int(rng.integers(0, 5))
    T = int(rng.integers(300, 2501))
    c = dict(renorm=0, drop=0, capacity=0, keep_num=9, keep_den=10, n_groups=0, topk_groups=0, route_mode=0,
             sel_bias_gate=0, sel_bias_steps=0, seq_len=0, n_shared=0, latent_proj=0,
             residual=int(rng.integers(0, 2)), act=int(rng.integers(0, 2)), act_dtype=1,
             router_dtype=int(rng.integers(0, 2)), d_ff=int(rng.choice([64, 128, 256])),
             zipf_s=float(rng.choice([0.0, 1.0])), tag=7000 + i)
    if kind == 0:
        Eh = int(rng.choice([8, 12, 16, 24, 32]))
        ng = int(rng.choice([g for g in (2, 4, 8) if Eh % g == 0]))
        k = int(rng.integers(1, 7))
        need = -(-k // (Eh // ng))
        dh = int(rng.choice([128, 256, 384]))
        c.update(n_heads=1, d_head=dh, d_model=dh, n_experts=Eh, top_k=k, n_groups=ng,
                 topk_groups=int(rng.integers(need, ng + 1)), drop=2, renorm=int(rng.integers(0, 2)),
                 n_shared=int(rng.integers(0, 3)))
    elif kind == 1:
        E = int(rng.integers(2, 33))
        dh = int(rng.choice([128, 256, 320]))
        c.update(n_heads=1, d_head=dh, d_model=dh, n_experts=E, top_k=1, route_mode=1, drop=1,
                 capacity=int(rng.integers(1, T + 10)))
    elif kind == 2:
        E = int(rng.integers(4, 65))
        L = int(rng.integers(16, 257))
        dh = int(rng.choice([128, 256]))
        c.update(n_heads=1, d_head=dh, d_model=dh, n_experts=E, top_k=int(rng.integers(1, min(E, 8) + 1)),
                 sel_bias_steps=5, sel_bias_gate=int(rng.integers(0, 2)), seq_len=L)
        T = max(L, T // L * L)
    elif kind == 3:
        H = int(rng.choice([2, 4, 8]))
        c.update(n_heads=H, d_head=int(rng.choice([64, 128, 256])), d_model=int(rng.choice([256, 512, 1024])),
                 n_experts=H * int(rng.integers(2, 17)), top_k=1, latent_proj=1, residual=1)
    else:
        H = int(rng.choice([2, 4]))
        Eh = int(rng.integers(2, 17))
        k = int(rng.integers(1, min(Eh, 8) + 1))
        drop = int(rng.integers(0, 3))
        c.update(n_heads=H, d_head=int(rng.choice([64, 128, 192, 256])), d_model=int(rng.choice([256, 512])),
                 n_experts=H * Eh, top_k=k, latent_proj=1, drop=drop,
                 capacity=int(rng.integers(1, -(-T * k // Eh) * 2)) if drop == 1 else 0)
    return MoEConfig(f"variant{i:03d}", T=T, **c)


# A few of each larger family run by default; MOE_RANDOM_SWEEP=N runs N of each.
N_SWEEP = int(os.environ.get("MOE_RANDOM_SWEEP", "0"))
LARGE = [draw_large(i) for i in range(max(N_SWEEP, 6))]
VARIANT = [draw_variant(i) for i in range(max(N_SWEEP, 10))]
# the forward keeping the routed pre-activations for the backward
KEPT = [draw(i) for i in range(max(N_SWEEP, 6))] + LARGE[:max(N_SWEEP, 6)]


def _dy(cfg):
    a = np.random.default_rng([77, cfg.tag]).standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    return bf16_bits_from_f32(a) if cfg.act_dtype == 1 else a


# the larger draws also ask for x_perm: the dispatch's row copy and the expert FFN on it
LAYER_CASES = [(c, False) for c in CASES + VARIANT] + [(c, True) for c in LARGE]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,xperm", LAYER_CASES, ids=[c.name + ("-xperm" if xp else "") for c, xp in LAYER_CASES])
def test_random_layer_forward_backward(cfg, xperm):
    check_layer(cfg, xperm=xperm)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", KEPT, ids=lambda c: c.name)
def test_random_layer_kept_preactivations(cfg):
    """The same checks with the forward keeping the routed pre-activations (io.gu) and
    the backward reading them (ignored by layers on the fused narrow-expert MLP)."""
    check_layer(cfg, keep=True)


def check_layer(cfg, keep=False, xperm=False):
    log(f"random {cfg}" + (" (pre-activations kept)" if keep else "") + (" (x_perm)" if xperm else ""))
    inp = generate(cfg, threads=1)
    out = oracle.forward(cfg, inp)
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = max(moe.moe_rows_upper_bound(cfg), 1)
    io = dict(logits=dev(out["logits"]), logits_mode=moe.MOE_LOGITS_LOAD, topk_idx=i32(T, K), topk_w=f32(T, K),
              demand=i32(E), counts=i32(E), offsets=i32(E + 1), row_of=i32(T, K), src_of=i32(Rm),
              y_perm=empty_act(cfg, Rm, cfg.d_head),
              aux_loss=f32(1) if cfg.n_heads == 1 else None,
              seq_loss=f32(T // cfg.seq_len) if cfg.seq_len else None,
              z=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None,
              o=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None,
              gu=empty_act(cfg, Rm, (2 if cfg.act == 1 else 1) * cfg.d_ff) if keep else None,
              x_perm=empty_act(cfg, Rm, cfg.d_head) if xperm else None)
    W = weights_dev(cfg, inp)
    x = dev(inp.x)
    y = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, W, x, y, io, moe.workspace(cfg))
    torch.cuda.synchronize()

    # choices: exact, or (selection bias) differing only at an oracle key near-tie
    idx = io["topk_idx"].cpu().numpy()
    diff = np.nonzero(np.any(idx != out["topk_idx"], axis=1))[0]
    if len(diff):
        assert cfg.sel_bias_steps > 0, f"choices differ at tokens {diff[:8]}"
        keys = out["p"] + np.asarray(inp.sel_bias, np.float64)[None, :]
        assert np.all(routing_margin(cfg, keys)[diff] < 1e-5), "choices differ away from a near-tie"
        log(f"  near-tie tokens: {len(diff)}")
    # the keep rule on the GPU's own choices and gates, exactly; where the
    # choices match the oracle's, keep decisions differ only at gate near-ties
    flips = check_keep(cfg, io, out, near_ties=len(diff) == 0)
    if len(flips):
        log(f"  keep decisions at gate near-ties: {len(flips)}")
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    if xperm:
        # every x_perm row is a bitwise copy of its source row (the head's slice of x or z)
        R = int(io["offsets"][-1])
        a = io["src_of"][:R].long()
        e_of = io["topk_idx"].reshape(-1).long()[a]
        src = (io["z"] if cfg.latent_proj else x).view(T, cfg.n_heads, cfg.d_head)
        want = src[a // K, e_of // cfg.e_per_head]
        bits = (lambda t: t.view(torch.int16)) if want.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
        assert torch.equal(bits(io["x_perm"][:R]), bits(want)), "x_perm rows"
    P = OB.params_of(inp)

    y_ref, _ = OB.forward_fixed(cfg, P, idx, kept)
    scale = max(np.max(np.abs(y_ref)), 1e-30)
    err = np.max(np.abs(f64(y) - y_ref))
    log(f"  y rel err {err / scale:.3g}")
    assert err <= tol(cfg) * scale
    if cfg.seq_len and len(diff) == 0:
        got = f64(io["seq_loss"])
        assert np.allclose(got, out["seq"], rtol=1e-5, atol=1e-7)

    lam = 0.5 if cfg.n_heads == 1 else 0.0
    sw = 0.3 if cfg.seq_len else 0.0
    dy_h = _dy(cfg)
    G = _grads(cfg)
    moe.moe_layer_bwd(cfg, W, _transposed(cfg, W), x, dev(dy_h), lam, io, G, moe.backward_workspace(cfg),
                      seq_weight=sw)
    torch.cuda.synchronize()
    # a latent layer's router and experts read z as the layer stores it (its activation
    # type): the oracle takes its own x W_in^T rounded the same way
    u = oracle.decode(act_round(cfg, OB._u(cfg, P))) if cfg.latent_proj else None
    ref = OB.backward(cfg, P, idx, kept, oracle.decode(dy_h), lam, sw, u=u)
    names = ["dx", "dw_router", "dw1", "dw2"] + (["dbias"] if inp.bias is not None else [])
    names += ["dw3"] if cfg.act == 1 else []
    if cfg.n_shared:
        names += ["dws1", "dws2"] + (["dws3"] if cfg.act == 1 else [])
    if cfg.latent_proj:
        names += ["dw_in", "dw_out"]
    # ReLU layers: a pre-activation near 0 may take the other side of the mask on the GPU
    ties, nties = relu_tie_allowance(cfg, P, idx, kept, oracle.decode(dy_h))
    if nties:
        log(f"  ReLU pre-activations near 0: {nties}")
    for n in names:
        got, want = f64(G[n]), ref[n]
        sc = max(np.max(np.abs(want)), 1e-30)
        if n == "dbias":
            # a sum over tokens of logit gradients, each within the bars: independent
            # rounding errors of its terms grow with their root sum of squares, which
            # a cancelling sum can fall far below
            sc = max(sc, np.max(np.sqrt(np.sum(ref["dl"] ** 2, axis=0))))
        e = np.max(np.abs(got - want)) if want.size else 0.0
        log(f"  {n:9s} rel err {e / sc:.3g}")
        assert np.all(np.isfinite(got)), n
        # router gradients are float32 throughout: an absolute floor covers a ~0 reference
        bound = tol(cfg) * sc + (1e-6 if n in ("dw_router", "dbias") else 0.0)
        if ties.get(n) is not None:
            assert np.all(np.abs(got - want) <= bound + ties[n]), n
        else:
            assert e <= bound, n


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES + VARIANT, ids=lambda c: c.name)
def test_random_route_compute(cfg):
    """moe_route computing its own scores: within 1e-5 * max|l| of the oracle's; choices differ only at near-ties."""
    log(f"random route COMPUTE {cfg.name}")
    inp = generate(cfg, threads=1)
    out = oracle.forward(cfg, inp)
    xin = bf16_bits_from_f32(out["z"].astype(np.float32)) if (cfg.latent_proj and cfg.act_dtype == 1) else (
        out["z"].astype(np.float32) if cfg.latent_proj else inp.x)
    ref = oracle.route(cfg, oracle.decode(xin), inp.w_router, inp.bias, sel_bias=inp.sel_bias)
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    idx, w, logits = i32(T, K), f32(T, K), f32(T, E)
    moe.moe_route(cfg, dev(xin), dev(inp.w_router), dev(inp.bias), logits, moe.MOE_LOGITS_COMPUTE_STORE, idx, w,
                  None, moe.workspace(cfg), sel_bias=dev(inp.sel_bias))
    torch.cuda.synchronize()
    l = logits.cpu().numpy().astype(np.float64)
    lmax = max(np.max(np.abs(ref["logits"])), 1e-30)
    err = np.max(np.abs(l - ref["logits"]))
    log(f"  scores rel err {err / lmax:.3g}")
    assert err <= 1e-5 * lmax
    got = idx.cpu().numpy()
    diff = np.nonzero(np.any(got != ref["topk_idx"], axis=1))[0]
    if len(diff):
        if inp.sel_bias is not None:
            margin = routing_margin(cfg, ref["p"] + np.asarray(inp.sel_bias, np.float64)[None, :])
            assert np.all(margin[diff] < 1e-5)
        else:
            margin = routing_margin(cfg, ref["logits"])
            assert np.all(margin[diff] <= 4 * err + 1e-30)
        log(f"  near-tie tokens: {len(diff)}")
    same = np.setdiff1d(np.arange(T), diff)
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64)[same] - ref["topk_w"][same]), initial=0.0) <= 1e-5
