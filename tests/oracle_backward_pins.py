"""Checks that pin the backward oracle (oracle/moe_backward.py) to facts outside itself.

What pins what:
  every gradient   central finite differences of L = <dy, y> + lam * l_aux
                   (float64, decisions frozen) along random directions, for
                   every parameter, on tiny configurations covering ReLU /
                   SwiGLU, renormalised gates, capacity and affinity drops,
                   group-limited routing, shared experts, the residual
                   switch, expert-choice routing, the balancing bias in and
                   out of the (renormalised) gate, several routing heads with
                   and without the latent projections (W_in and W_out
                   perturbed too), and the aux-loss term alone
  forward_fixed    equals the main oracle's layer output (which takes its
                   probabilities from float32-rounded logits) to 1e-5
  special cases    one expert with top-1: p = g = 1, so no gradient reaches
                   the router; gradients are linear in dy; with dy = 0 only
                   the aux term moves the router
Each check raises AssertionError on failure; test_oracle_backward.py calls them
directly and against planted mistakes.
"""
import numpy as np

from moe_inputs import MoEConfig, generate

RELU, SWIGLU = 0, 1


def _mods():
    import oracle.moe_backward as B
    import oracle.moe_oracle as O
    return B, O


def tiny_cfgs():
    base = MoEConfig("bwd_tiny", T=12, d_model=16, n_heads=1, d_head=16, n_experts=4, top_k=2, d_ff=8,
                     act_dtype=0, router_dtype=0, tag=60)
    return [
        base.with_(name="bwd_relu", act=RELU),
        base.with_(name="bwd_swiglu_renorm", renorm=1),
        base.with_(name="bwd_capacity_shared", drop=1, capacity=4, n_shared=2),
        base.with_(name="bwd_affinity_groups", drop=2, keep_num=2, keep_den=3, n_groups=2, topk_groups=1,
                   n_experts=6, top_k=2),
        base.with_(name="bwd_no_residual_zipf", residual=0, zipf_s=1.0, top_k=3),
        base.with_(name="bwd_expert_choice", route_mode=1, drop=1, capacity=5),
        base.with_(name="bwd_selbias_in_gate", sel_bias_steps=40, sel_bias_gate=1, n_shared=1),
        base.with_(name="bwd_selbias_renorm", sel_bias_steps=40, renorm=1),
        base.with_(name="bwd_selbias_in_gate_renorm", sel_bias_steps=40, sel_bias_gate=1, renorm=1),
        MoEConfig("bwd_multihead_latent", T=10, d_model=24, n_heads=2, d_head=8, n_experts=6, top_k=1, d_ff=8,
                  latent_proj=1, zipf_s=1.0, act_dtype=0, router_dtype=0, tag=61),
        MoEConfig("bwd_multihead_renorm_relu", T=11, d_model=16, n_heads=2, d_head=8, n_experts=4, top_k=2,
                  renorm=1, d_ff=8, act=RELU, act_dtype=0, router_dtype=0, tag=62),
        base.with_(name="bwd_one_expert", n_experts=1, top_k=1),
    ]


def _setup(cfg, seed=0):
    B, O = _mods()
    inp = generate(cfg)
    out = O.forward(cfg, inp)
    P = B.params_of(inp)
    rng = np.random.default_rng([seed, cfg.tag])
    dy = rng.standard_normal((cfg.T, cfg.d_model))
    return inp, out, P, dy


def _names(cfg, P):
    n = ["x", "w_router", "w1", "w2"]
    if P["bias"] is not None:
        n.append("bias")
    if P["w3"] is not None:
        n.append("w3")
    if cfg.n_shared:
        n += ["ws1", "ws2"] + (["ws3"] if P["ws3"] is not None else [])
    if cfg.latent_proj:
        n += ["w_in", "w_out"]
    return n


_GRAD = dict(x="dx", w_router="dw_router", bias="dbias", w1="dw1", w3="dw3", w2="dw2",
             ws1="dws1", ws3="dws3", ws2="dws2", w_in="dw_in", w_out="dw_out")


def _fd_check(cfg, lam, dy_scale=1.0, eps=1e-6, tol=1e-6, seq_w=0.0):
    B, O = _mods()
    inp, out, P, dy = _setup(cfg)
    dy = dy * dy_scale
    idx, kept = out["topk_idx"], out["kept"]
    G = B.backward(cfg, P, idx, kept, dy, lam, seq_w)
    rng = np.random.default_rng([7, cfg.tag])
    for name in _names(cfg, P):
        v = rng.standard_normal(P[name].shape)
        Pp = dict(P); Pp[name] = P[name] + eps * v
        Pm = dict(P); Pm[name] = P[name] - eps * v
        _, Lp = B.forward_fixed(cfg, Pp, idx, kept, lam, dy, seq_w)
        _, Lm = B.forward_fixed(cfg, Pm, idx, kept, lam, dy, seq_w)
        fd = (Lp - Lm) / (2 * eps)
        an = float(np.sum(G[_GRAD[name]] * v))
        assert abs(fd - an) <= tol * max(1.0, abs(an)), f"{cfg.name} lam={lam} d{name}: fd {fd} vs {an}"


def _lam(cfg, lam):
    """The aux loss exists for one routing head only."""
    return lam if cfg.n_heads == 1 else 0.0


def check_fd_all():
    for cfg in tiny_cfgs():
        _fd_check(cfg, 0.0)
        if cfg.n_heads == 1:
            _fd_check(cfg, 0.37)


def check_fd_seq_term():
    """The sequence-wise balance term, with and without the aux term, and alone (dy = 0)."""
    base = tiny_cfgs()[1]
    for cfg in (base.with_(name="bwd_seq3", T=12, seq_len=4), base.with_(name="bwd_seq_whole", seq_len=12),
                tiny_cfgs()[3].with_(name="bwd_seq_groups", seq_len=6)):
        _fd_check(cfg, 0.0, seq_w=0.8)
        _fd_check(cfg, 0.3, seq_w=0.8)
        _fd_check(cfg, 0.0, dy_scale=0.0, seq_w=1.0)


def check_seq_term_whole_batch_equals_aux():
    """One sequence over the whole batch: the term equals l_aux, so its gradient equals the aux gradient."""
    B, O = _mods()
    cfg = tiny_cfgs()[2].with_(name="bwd_seq_eq_aux", seq_len=12)
    inp, out, P, dy = _setup(cfg)
    idx, kept = out["topk_idx"], out["kept"]
    ga = B.backward(cfg, P, idx, kept, dy, 0.7, 0.0)
    gs = B.backward(cfg, P, idx, kept, dy, 0.0, 0.7)
    for k in ("dx", "dw_router", "dbias", "dl"):
        assert np.allclose(ga[k], gs[k], rtol=1e-12, atol=1e-15), k


def check_fd_aux_only():
    # dy = 0: only the aux term has a gradient, and only through the router
    for cfg in tiny_cfgs()[:3]:
        _fd_check(cfg, 1.0, dy_scale=0.0)


def check_forward_fixed_matches_oracle():
    B, O = _mods()
    for cfg in tiny_cfgs():
        inp, out, P, dy = _setup(cfg)
        y, _ = B.forward_fixed(cfg, P, out["topk_idx"], out["kept"])
        ref = out["y"]
        assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref)), cfg.name


def check_special_cases():
    B, O = _mods()
    cfg = tiny_cfgs()[-1]  # one expert, top-1
    inp, out, P, dy = _setup(cfg)
    G = B.backward(cfg, P, out["topk_idx"], out["kept"], dy, 0.5)
    assert np.all(G["dl"] == 0) and np.all(G["dw_router"] == 0) and np.all(G["dbias"] == 0)
    # linear in dy (lam = 0)
    for cfg in tiny_cfgs()[:3]:
        inp, out, P, dy = _setup(cfg)
        g1 = B.backward(cfg, P, out["topk_idx"], out["kept"], dy, 0.0)
        g2 = B.backward(cfg, P, out["topk_idx"], out["kept"], 2.0 * dy, 0.0)
        for k in ("dx", "dw_router", "dw1", "dw2"):
            assert np.allclose(g2[k], 2.0 * g1[k], rtol=1e-12, atol=1e-12), (cfg.name, k)
    # dy = 0: no expert weight moves, the router does (through the aux term)
    cfg = tiny_cfgs()[1]
    inp, out, P, dy = _setup(cfg)
    G = B.backward(cfg, P, out["topk_idx"], out["kept"], np.zeros_like(dy), 1.0)
    assert np.all(G["dw1"] == 0) and np.all(G["dw2"] == 0) and np.any(G["dw_router"] != 0)


def check_restricted_forms():
    """backward_tokens and backward_expert (used at full size) equal the full backward."""
    B, O = _mods()
    for cfg in tiny_cfgs():
        inp, out, P, dy = _setup(cfg)
        idx, kept = out["topk_idx"], out["kept"]
        lam = _lam(cfg, 0.37)
        G = B.backward(cfg, P, idx, kept, dy, lam)
        toks = np.arange(0, cfg.T, 3)
        dx = B.backward_tokens(cfg, P, idx, kept, dy, lam, toks, out["demand"])
        assert np.allclose(dx, G["dx"][toks], rtol=1e-10, atol=1e-12), cfg.name
        for e in range(cfg.n_experts):
            dW1, dW3, dW2 = B.backward_expert(cfg, P, e, idx, kept, dy)
            assert np.allclose(dW1, G["dw1"][e], rtol=1e-10, atol=1e-12), (cfg.name, e)
            assert np.allclose(dW2, G["dw2"][e], rtol=1e-10, atol=1e-12), (cfg.name, e)
            if dW3 is not None:
                assert np.allclose(dW3, G["dw3"][e], rtol=1e-10, atol=1e-12), (cfg.name, e)
            hid = np.arange(1, cfg.d_ff, 3)
            h1, h3, h2 = B.backward_expert(cfg, P, e, idx, kept, dy, hidden=hid)
            assert np.allclose(h1, G["dw1"][e][hid], rtol=1e-10, atol=1e-12), (cfg.name, e)
            assert np.allclose(h2, G["dw2"][e][:, hid], rtol=1e-10, atol=1e-12), (cfg.name, e)


ALL = [check_fd_all, check_fd_seq_term, check_seq_term_whole_batch_equals_aux, check_fd_aux_only, check_forward_fixed_matches_oracle, check_special_cases,
       check_restricted_forms]
