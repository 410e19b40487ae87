"""Backward at the full workload sizes, in the launch configuration the benchmark times,
against the float64 backward oracle.  One-head workloads on samples it evaluates cheaply:
dx of sampled tokens (a token's input gradient needs only its own experts and the
demand counts), and the weight gradients of one expert restricted to sampled hidden
units (they decompose over hidden units).  Router gradients: every token's logit
gradient sums to zero over the experts (softmax Jacobian), so sum_e dbias_e and
every column sum of dW_router vanish.  The multi-head latent workload's experts are
small, so the oracle's whole backward runs and every gradient is compared.  Plus
finiteness and bitwise reproducibility.  The workloads whose routed experts run the
grouped GEMM run twice: recomputing the gate/up products, and (as the benchmark times
them) with the forward keeping the pre-activations (io.gu) for the backward.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.moe_backward as OB
import routing_dispatch_expert_router_amd as moe
from moe_inputs import CONFIGS, bf16_bits_from_f32
from tests.gpu_util import log, dev, f64, tol, weights_dev, cached_inputs

pytestmark = pytest.mark.gpu

FULL = CONFIGS[1:]
# (workload, pre-activations kept): kept only where the routed experts run the grouped GEMM
CASES = [(c, False) for c in FULL] + [(c, True) for c in FULL if c.act_dtype == 0 or c.d_head not in (64, 128, 256)]


def _lam(cfg):
    """Aux weight: the aux loss is defined for one routing head."""
    return 0.01 if cfg.n_heads == 1 else 0.0


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cfg,keep", CASES, ids=[c.name + ("-kept" if k else "") for c, k in CASES])
def test_fullsize_backward(cfg, keep):
    log(f"full-size backward {cfg.name}" + (" (pre-activations kept)" if keep else ""))
    inp = cached_inputs(cfg)
    T, K, E, dh, F, d = cfg.T, cfg.k_total, cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
    Rm = moe.moe_rows_upper_bound(cfg)
    adt = torch.bfloat16
    m = 2 if cfg.act == 1 else 1
    fs = cfg.n_shared * F
    e_ = lambda *s, dt=adt: torch.empty(*s, dtype=dt, device="cuda")
    io = dict(logits=e_(T, E, dt=torch.float32), logits_mode=moe.MOE_LOGITS_COMPUTE_STORE,
              topk_idx=e_(T, K, dt=torch.int32), topk_w=e_(T, K, dt=torch.float32), demand=e_(E, dt=torch.int32),
              counts=e_(E, dt=torch.int32), offsets=e_(E + 1, dt=torch.int32), row_of=e_(T, K, dt=torch.int32),
              src_of=e_(Rm, dt=torch.int32), y_perm=e_(Rm, dh),
              z=e_(T, cfg.d_latent) if cfg.latent_proj else None, o=e_(T, cfg.d_latent) if cfg.latent_proj else None,
              gu=e_(max(Rm, 1), m * F) if keep else None)
    W = weights_dev(cfg, inp)
    x = dev(inp.x)
    y = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, W, x, y, io, moe.workspace(cfg))
    D = cfg.d_latent
    wt = dict(w13t=e_(E, dh, m * F), w2t=e_(E, F, dh), ws13t=e_(d, m * fs) if fs else None,
              ws2t=e_(fs, d) if fs else None, w_in_t=e_(d, D) if cfg.latent_proj else None,
              w_out_t=e_(D, d) if cfg.latent_proj else None)
    moe.moe_transpose_weights(cfg, W, wt)
    rng = np.random.default_rng([5, cfg.tag])
    dy_h = bf16_bits_from_f32(rng.standard_normal((T, d)).astype(np.float32))
    dy = dev(dy_h)

    def grads():
        return dict(dx=e_(T, d), dw_router=e_(E, dh, dt=torch.float32), dbias=e_(E, dt=torch.float32),
                    dw1=e_(E, F, dh), dw3=e_(E, F, dh) if cfg.act == 1 else None, dw2=e_(E, dh, F),
                    dws1=e_(fs, d) if fs else None, dws3=e_(fs, d) if (fs and cfg.act == 1) else None,
                    dws2=e_(d, fs) if fs else None, dw_in=e_(D, d) if cfg.latent_proj else None,
                    dw_out=e_(d, D) if cfg.latent_proj else None)

    ws = moe.backward_workspace(cfg)
    G1, G2 = grads(), grads()
    log("  GPU backward x2")
    LAM = _lam(cfg)
    moe.moe_layer_bwd(cfg, W, wt, x, dy, LAM, io, G1, ws)
    moe.moe_layer_bwd(cfg, W, wt, x, dy, LAM, io, G2, ws)
    torch.cuda.synchronize()
    for k in G1:
        if G1[k] is not None:
            assert torch.isfinite(G1[k].float()).all(), k
            assert torch.equal(_bits(G1[k]), _bits(G2[k])), k
    # router gradients: zero sums over experts
    db = G1["dbias"].double()
    assert abs(float(db.sum())) <= 1e-4 * float(db.abs().sum())
    dwr = G1["dw_router"].double()
    assert float(dwr.sum(0).abs().max()) <= 1e-4 * float(dwr.abs().sum(0).max())
    # sampled tokens: dx
    P = OB.params_of(inp)
    idx = io["topk_idx"].cpu().numpy()
    kept = io["row_of"].cpu().numpy().reshape(-1) >= 0
    demand = io["demand"].cpu().numpy()
    dy64 = oracle.decode(dy_h)
    if cfg.latent_proj:
        log("  oracle: the whole backward")
        ref = OB.backward(cfg, P, idx, kept, dy64, LAM)
        names = ["dx", "dw_router", "dbias", "dw1", "dw2", "dw_in", "dw_out"] + (["dw3"] if cfg.act == 1 else [])
        for k in names:
            got, want = f64(G1[k]), ref[k]
            scale = np.max(np.abs(want))
            err = np.max(np.abs(got - want))
            log(f"  {k:10s} rel err {err / scale:.3g}")
            assert err <= tol(cfg) * scale, k
        return
    toks = np.linspace(0, T - 1, 6).astype(np.int64)
    log("  oracle: sampled tokens")
    ref = OB.backward_tokens(cfg, P, idx, kept, dy64, LAM, toks, demand)
    got = f64(G1["dx"])[toks]
    err = np.max(np.abs(got - ref))
    log(f"  dx (sampled tokens) rel err {err / np.max(np.abs(ref)):.3g}")
    assert err <= tol(cfg) * np.max(np.abs(ref))
    # one expert, sampled hidden units
    counts = io["counts"].cpu().numpy()
    e = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
    hid = np.linspace(0, F - 1, 32).astype(np.int64)
    log(f"  oracle: expert {e} ({counts[e]} rows), 32 hidden units")
    r1, r3, r2 = OB.backward_expert(cfg, P, e, idx, kept, dy64, hidden=hid)
    hid_t = torch.from_numpy(hid).cuda()
    for name, got_t, want in (("dw1", G1["dw1"][e][hid_t], r1), ("dw2", G1["dw2"][e][:, hid_t], r2),
                              ("dw3", G1["dw3"][e][hid_t] if r3 is not None else None, r3)):
        if want is None:
            continue
        g = f64(got_t)
        err = np.max(np.abs(g - want))
        log(f"  {name} (expert {e}) rel err {err / np.max(np.abs(want)):.3g}")
        assert err <= tol(cfg) * np.max(np.abs(want)), name
