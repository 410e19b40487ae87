"""GPU parity of the routing variants against the CPU oracle.

Expert-choice routing, the selection-only balancing bias (in or out of the
gate, with group-limited selection), the per-sequence balance statistic and
the bias update.  Bars as for the plain router: with the oracle's float32
scores loaded, indices, counts and the permutation bit-exact (the balancing
bias's keys p + b come from the GPU's own exp, so a token whose oracle key
margin is below 1e-6 may differ and is reported); gates within 1e-6; the
sequence statistic within 1e-5 relative; the bias update bitwise; the layer
output within 1e-4 / 2e-2 of max|y_ref| (float32 / bf16 layers).  Full-size
layers are checked on a sample of tokens.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import oracle.moe_backward as OB
import routing_dispatch_expert_router_amd as moe
from moe_inputs import SMALL_VARIANTS, VARIANTS, generate
from tests.gpu_util import log, dev, f64, empty_act, i32, f32, cached_inputs, tol, weights_dev, check_keep

pytestmark = pytest.mark.gpu

IDS = [c.name for c in SMALL_VARIANTS]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@functools.lru_cache(maxsize=8)
def oracle_out(cfg):
    return oracle.forward(cfg, cached_inputs(cfg), want_xperm=True)


def key_margin(cfg, p, sel_bias):
    """Per token, the smallest gap between keys p + b that decides the top-k (and the group choice)."""
    keys = oracle.biased_keys(p, sel_bias).astype(np.float64)
    T, E, k = keys.shape[0], keys.shape[1], cfg.top_k
    s = np.sort(keys, axis=1)[:, ::-1]
    gap = s[:, k - 1] - s[:, k] if k < E else np.full(T, np.inf)
    if cfg.n_groups:
        g = np.sort(keys.reshape(T, cfg.n_groups, -1).max(axis=2), axis=1)[:, ::-1]
        if cfg.topk_groups < cfg.n_groups:
            gap = np.minimum(gap, g[:, cfg.topk_groups - 1] - g[:, cfg.topk_groups])
    return gap


def _route(cfg, out, inp):
    T, K = cfg.T, cfg.k_total
    ws = moe.workspace(cfg)
    idx, w = i32(T, K), f32(T, K)
    aux = f32(1)
    seq = f32(T // cfg.seq_len) if cfg.seq_len else None
    moe.moe_route(cfg, None, None, None, dev(out["logits"]), moe.MOE_LOGITS_LOAD, idx, w, aux, ws,
                  sel_bias=dev(inp.sel_bias), seq_loss=seq)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), f64(w), float(aux.item()), (None if seq is None else f64(seq))


@pytest.mark.parametrize("cfg", SMALL_VARIANTS, ids=IDS)
def test_variant_route_load(cfg):
    log(f"variant route LOAD {cfg.name}")
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    idx, w, aux, seq = _route(cfg, out, inp)
    ok = np.ones(cfg.T, bool)
    if inp.sel_bias is not None:
        diff = np.nonzero(np.any(idx != out["topk_idx"], axis=1))[0]
        margin = key_margin(cfg, out["p"], inp.sel_bias)
        log(f"  tokens routed differently: {len(diff)} (smallest key margin {margin.min():.3g})")
        assert np.all(margin[diff] < 1e-6), "routing differs at a token whose keys are not a near-tie"
        ok[diff] = False
    else:
        assert np.array_equal(idx, out["topk_idx"])
    assert np.max(np.abs(w[ok] - out["topk_w"][ok])) <= 1e-6
    assert abs(aux - out["aux"]) <= 1e-5 * max(1.0, abs(out["aux"]))
    if cfg.seq_len:
        log(f"  sequence statistic {seq} vs {out['seq']}")
        assert np.all(np.abs(seq - out["seq"]) <= 1e-5 * np.maximum(1.0, np.abs(out["seq"])))


@pytest.mark.parametrize("cfg", SMALL_VARIANTS, ids=IDS)
def test_variant_dispatch_bitexact(cfg):
    log(f"variant dispatch {cfg.name}")
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = moe.moe_rows_upper_bound(cfg)
    ws = moe.workspace(cfg)
    demand, counts, offsets = i32(E), i32(E), i32(E + 1)
    row_of, src_of = i32(T, K), i32(Rm)
    xp = empty_act(cfg, Rm, cfg.d_head)
    moe.moe_dispatch(cfg, dev(out["topk_idx"]), dev(out["topk_w32"]), dev(inp.x), demand, counts, offsets, row_of,
                     src_of, xp, ws)
    torch.cuda.synchronize()
    R = int(out["offsets"][-1])
    assert np.array_equal(demand.cpu().numpy(), out["demand"])
    assert np.array_equal(counts.cpu().numpy(), out["counts"])
    assert np.array_equal(offsets.cpu().numpy(), out["offsets"])
    assert np.array_equal(row_of.cpu().numpy(), out["row_of"])
    assert np.array_equal(src_of.cpu().numpy()[:R], out["src_of"])
    assert np.array_equal(f64(xp[:R]), oracle.decode(inp.x)[out["src_of"] // K])
    if cfg.route_mode == 1:
        assert np.all(out["counts"] == min(cfg.capacity, cfg.T))


def _layer(cfg, inp, logits, with_xperm=False):
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = max(moe.moe_rows_upper_bound(cfg), 1)
    io = dict(logits=dev(logits), logits_mode=moe.MOE_LOGITS_LOAD, topk_idx=i32(T, K), topk_w=f32(T, K),
              demand=i32(E), counts=i32(E), offsets=i32(E + 1), row_of=i32(T, K), src_of=i32(Rm),
              y_perm=empty_act(cfg, Rm, cfg.d_head), aux_loss=f32(1),
              seq_loss=f32(T // cfg.seq_len) if cfg.seq_len else None,
              x_perm=empty_act(cfg, Rm, cfg.d_head) if with_xperm else None)
    W = weights_dev(cfg, inp)
    x = dev(inp.x)
    y = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, W, x, y, io, moe.workspace(cfg))
    torch.cuda.synchronize()
    return y, io, W, x


@pytest.mark.parametrize("cfg", SMALL_VARIANTS, ids=IDS)
def test_variant_layer(cfg):
    log(f"variant layer {cfg.name}")
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    y, io, _, _ = _layer(cfg, inp, out["logits"])
    idx = io["topk_idx"].cpu().numpy()
    diff = np.nonzero(np.any(idx != out["topk_idx"], axis=1))[0]
    if inp.sel_bias is None:
        assert len(diff) == 0
    else:
        margin = key_margin(cfg, out["p"], inp.sel_bias)
        log(f"  tokens routed differently: {len(diff)}")
        assert np.all(margin[diff] < 1e-6), "routing differs at a token whose keys are not a near-tie"
    # keep rule exact on the GPU's gates; differences from the oracle's own keep only at near-ties
    if len(diff) == 0:
        flips = check_keep(cfg, io, out)
        log(f"  keep decisions that differ from the oracle's: {len(flips)}")
    # every token against the oracle's output for the GPU's own decisions
    import oracle.moe_backward as OB
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    ref, _ = OB.forward_fixed(cfg, OB.params_of(inp), idx, kept)
    err = np.max(np.abs(f64(y) - ref))
    log(f"  max err {err:.3g} (rel {err / np.max(np.abs(ref)):.3g})")
    assert err <= tol(cfg) * np.max(np.abs(ref))
    if cfg.seq_len:
        seq = f64(io["seq_loss"])
        assert np.all(np.abs(seq - out["seq"]) <= 1e-5 * np.maximum(1.0, np.abs(out["seq"])))


@pytest.mark.parametrize("cfg", SMALL_VARIANTS, ids=IDS)
def test_variant_gather_equals_xperm(cfg):
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    y1, io1, _, _ = _layer(cfg, inp, out["logits"], with_xperm=True)
    y2, io2, _, _ = _layer(cfg, inp, out["logits"], with_xperm=False)
    b = (lambda t: t.view(torch.int16)) if y1.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(b(y1), b(y2))


def test_sel_bias_update_bitwise():
    cfg = SMALL_VARIANTS[1]
    rng = np.random.default_rng(3)
    for trial in range(3):
        load = rng.integers(0, 400, size=cfg.n_experts).astype(np.int32)
        if trial == 1:
            load[:] = 37  # every expert at the mean: unchanged
        b = (rng.integers(-20, 21, size=cfg.n_experts) * 0.001).astype(np.float32)
        ref = oracle.sel_bias_update(b, load, 0.001)
        bd = dev(b.copy())
        moe.moe_sel_bias_update(cfg, dev(load), bd, 0.001)
        torch.cuda.synchronize()
        assert np.array_equal(bd.cpu().numpy().view(np.uint32), ref.view(np.uint32)), trial


def test_sel_bias_update_multihead():
    """Per head: each head's experts compare against that head's own mean load."""
    from moe_inputs import SMALL
    cfg = SMALL[4]
    H, Eh = cfg.n_heads, cfg.e_per_head
    rng = np.random.default_rng(4)
    load = rng.integers(0, 50, size=cfg.n_experts).astype(np.int32)
    b = np.zeros(cfg.n_experts, np.float32)
    ref = np.concatenate([oracle.sel_bias_update(b[h * Eh:(h + 1) * Eh], load[h * Eh:(h + 1) * Eh], 0.001)
                          for h in range(H)])
    bd = dev(b.copy())
    moe.moe_sel_bias_update(cfg, dev(load), bd, 0.001)
    torch.cuda.synchronize()
    assert np.array_equal(bd.cpu().numpy(), ref)


# ------------------------------------------------------------------ full size (sampled tokens)
SAMPLE = 24


@pytest.mark.parametrize("cfg", VARIANTS, ids=[c.name for c in VARIANTS])
def test_variant_fullsize(cfg):
    log(f"variant full-size {cfg.name}: inputs")
    inp = cached_inputs(cfg)
    toks = np.linspace(0, cfg.T - 1, SAMPLE).astype(np.int64)
    log("  oracle (routing and keep of every token, outputs of the sample)")
    out = oracle.forward(cfg, inp, tokens=toks)
    log("  GPU layer, scores loaded")
    y, io, _, _ = _layer(cfg, inp, out["logits"])
    idx = io["topk_idx"].cpu().numpy()
    row_of = io["row_of"].cpu().numpy()
    if inp.sel_bias is None:
        assert np.array_equal(idx, out["topk_idx"])
        flips = check_keep(cfg, io, out)
        log(f"  keep decisions that differ from the oracle's: {len(flips)}")
        assert np.array_equal(io["counts"].cpu().numpy(), out["counts"])
    else:
        diff = np.nonzero(np.any(idx != out["topk_idx"], axis=1))[0]
        margin = key_margin(cfg, out["p"], inp.sel_bias)
        log(f"  tokens routed differently: {len(diff)}")
        assert np.all(margin[diff] < 1e-6)
        assert np.array_equal(io["demand"].cpu().numpy().sum(), out["demand"].sum())
    ok = np.all(idx[toks] == out["topk_idx"][toks], axis=1) & \
        np.all((row_of[toks] >= 0) == (out["row_of"][toks] >= 0), axis=1)
    got, ref = f64(y)[toks], out["y"]
    err = np.max(np.abs(got[ok] - ref[ok]))
    log(f"  sampled rows ({int(ok.sum())} of {len(toks)}): max err {err:.3g}, rel {err / np.max(np.abs(ref)):.3g}")
    assert ok.sum() >= len(toks) - 1
    assert err <= tol(cfg) * np.max(np.abs(ref))
    if cfg.seq_len:
        seq = f64(io["seq_loss"])
        log(f"  sequence statistic {seq} vs {out['seq']}")
        assert np.all(np.abs(seq - out["seq"]) <= 1e-5 * np.maximum(1.0, np.abs(out["seq"])))


# ------------------------------------------------------------------ backward
@pytest.mark.parametrize("cfg", SMALL_VARIANTS, ids=IDS)
def test_variant_backward(cfg):
    log(f"variant backward {cfg.name}")
    from tests.test_gpu_backward import _transposed, _grads, _dy
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    y, io, W, x = _layer(cfg, inp, out["logits"])
    io["logits"] = dev(out["logits"])
    wt = _transposed(cfg, W)
    dy_h = _dy(cfg)
    G = _grads(cfg)
    lam = 0.5
    sw = 2.0 if cfg.seq_len else 0.0  # the sequence-wise balance term, where the layer reports it
    moe.moe_layer_bwd(cfg, W, wt, x, dev(dy_h), lam, io, G, moe.backward_workspace(cfg), seq_weight=sw)
    torch.cuda.synchronize()
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    P = OB.params_of(inp)
    ref = OB.backward(cfg, P, io["topk_idx"].cpu().numpy(), kept, oracle.decode(dy_h), lam, sw)
    names = ["dx", "dw_router", "dbias", "dw1", "dw2"] + (["dw3"] if cfg.act == 1 else [])
    if cfg.n_shared:
        names += ["dws1", "dws2"] + (["dws3"] if cfg.act == 1 else [])
    for k in names:
        got, want = f64(G[k]), ref[k]
        scale = max(np.max(np.abs(want)), 1e-30)
        err = np.max(np.abs(got - want))
        log(f"  {k:10s} rel err {err / scale:.3g}")
        assert err <= tol(cfg) * scale, k


def test_sequence_term_router_gradient():
    """The sequence term alone (dy = 0, no aux): only the router moves, and it matches the oracle."""
    cfg = SMALL_VARIANTS[1]
    from tests.test_gpu_backward import _transposed, _grads
    inp = cached_inputs(cfg)
    out = oracle_out(cfg)
    y, io, W, x = _layer(cfg, inp, out["logits"])
    G = _grads(cfg)
    dy = torch.zeros_like(x)
    moe.moe_layer_bwd(cfg, W, _transposed(cfg, W), x, dy, 0.0, io, G, moe.backward_workspace(cfg), seq_weight=1.0)
    torch.cuda.synchronize()
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    ref = OB.backward(cfg, OB.params_of(inp), io["topk_idx"].cpu().numpy(), kept,
                      np.zeros((cfg.T, cfg.d_model)), 0.0, 1.0)
    assert float(G["dw1"].float().abs().max()) == 0.0
    for k in ("dw_router", "dbias", "dx"):
        got, want = f64(G[k]), ref[k]
        scale = np.max(np.abs(want))
        assert scale > 0, k
        assert np.max(np.abs(got - want)) <= 2e-2 * scale, k


# ------------------------------------------------------------------ edge cases
def _edge_variants():
    from moe_inputs import MoEConfig
    base = MoEConfig("edge_var", T=37, d_model=128, n_heads=1, d_head=128, n_experts=4, top_k=2, d_ff=128,
                     drop=1, capacity=9, route_mode=1, tag=80)
    return [
        base.with_(name="edge_ec_capacity0_shared", capacity=0, n_shared=1),
        base.with_(name="edge_ec_capacity_over_T", capacity=50),
        base.with_(name="edge_ec_T1", T=1, capacity=1),
        base.with_(name="edge_ec_E1_relu_f32", n_experts=1, top_k=1, capacity=20, act=0, act_dtype=0,
                   router_dtype=0),
        base.with_(name="edge_bias_seq_T1", T=1, route_mode=0, drop=0, capacity=0, sel_bias_steps=5, seq_len=1),
        base.with_(name="edge_bias_seq_whole", route_mode=0, drop=0, capacity=0, sel_bias_steps=5,
                   sel_bias_gate=1, seq_len=37, top_k=4),
    ]


@pytest.mark.parametrize("cfg", _edge_variants(), ids=lambda c: c.name)
def test_variant_edges(cfg):
    log(f"variant edge {cfg.name}")
    inp = generate(cfg)
    out = oracle.forward(cfg, inp, want_xperm=True)
    y, io, _, _ = _layer(cfg, inp, out["logits"])
    assert np.array_equal(io["counts"].cpu().numpy(), out["counts"])
    assert np.array_equal(io["row_of"].cpu().numpy(), out["row_of"])
    got, ref = f64(y), out["y"]
    err = np.max(np.abs(got - ref))
    log(f"  max err {err:.3g}")
    assert err <= tol(cfg) * max(np.max(np.abs(ref)), 1e-30)
    if cfg.seq_len:
        seq = f64(io["seq_loss"])
        assert np.all(np.abs(seq - out["seq"]) <= 1e-5 * np.maximum(1.0, np.abs(out["seq"])))
    # the backward on the same decisions
    from tests.test_gpu_backward import _transposed, _grads, _dy
    W = weights_dev(cfg, inp)
    x = dev(inp.x)
    G = _grads(cfg)
    dy_h = _dy(cfg)
    moe.moe_layer_bwd(cfg, W, _transposed(cfg, W), x, dev(dy_h), 0.5, io, G, moe.backward_workspace(cfg))
    torch.cuda.synchronize()
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    ref = OB.backward(cfg, OB.params_of(inp), io["topk_idx"].cpu().numpy(), kept, oracle.decode(dy_h), 0.5)
    for k in ["dx", "dw_router", "dbias", "dw1", "dw2"] + (["dws1", "dws2"] if cfg.n_shared else []):
        got, want = f64(G[k]), ref[k]
        # floor 1e-6: with expert choice every expert's aux load is T, so when no gate
        # gradient reaches the router its dp is constant and the softmax Jacobian cancels
        # it exactly; both sides then hold only rounding (float64 ~1e-18, float32 ~1e-9)
        scale = max(np.max(np.abs(want)), 1e-6)
        assert np.all(np.isfinite(got)), k
        assert np.max(np.abs(got - want)) <= tol(cfg) * scale, k
