"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

For each full-size workload: the whole layer runs on the GPU with the oracle's
float32 scores loaded (routing, counts and the permutation must then be
bit-exact), and also free-running (scores within 1e-5*max|l| where the router
input is bit-identical on both sides; routing may differ only at near-ties).
Output rows are compared with the float64 oracle on a sample of tokens the
oracle evaluates one by one; x_perm rows are checked bitwise on a row sample.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_router_amd as moe
from moe_inputs import CONFIGS
from tests.gpu_util import log, dev, f64, tol, weights_dev, routing_margin, cached_inputs, check_keep

pytestmark = pytest.mark.gpu

FULL = CONFIGS[1:]
SAMPLE = 24


def _run(cfg, inp, logits_load, with_xperm=True):
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = moe.moe_rows_upper_bound(cfg)
    adt = torch.bfloat16 if cfg.act_dtype == 1 else torch.float32
    io = dict(topk_idx=torch.empty(T, K, dtype=torch.int32, device="cuda"),
              topk_w=torch.empty(T, K, dtype=torch.float32, device="cuda"),
              demand=torch.empty(E, dtype=torch.int32, device="cuda"),
              counts=torch.empty(E, dtype=torch.int32, device="cuda"),
              offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
              row_of=torch.empty(T, K, dtype=torch.int32, device="cuda"),
              src_of=torch.empty(Rm, dtype=torch.int32, device="cuda"),
              x_perm=torch.empty(Rm, cfg.d_head, dtype=adt, device="cuda") if with_xperm else None,
              z=torch.empty(T, cfg.d_latent, dtype=adt, device="cuda") if cfg.latent_proj else None)
    if logits_load is not None:
        io["logits"] = dev(logits_load)
        io["logits_mode"] = moe.MOE_LOGITS_LOAD
    else:
        io["logits"] = torch.empty(T, E, dtype=torch.float32, device="cuda")
        io["logits_mode"] = moe.MOE_LOGITS_COMPUTE_STORE
    x = dev(inp.x)
    y = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, weights_dev(cfg, inp), x, y, io, moe.workspace(cfg))
    torch.cuda.synchronize()
    return y, io, x


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fullsize_layer(cfg):
    log(f"full-size {cfg.name}: inputs")
    inp = cached_inputs(cfg)
    toks = np.linspace(0, cfg.T - 1, SAMPLE).astype(np.int64)
    log("  oracle (routing of every token, outputs of the sample)")
    out = oracle.forward(cfg, inp, tokens=toks)
    log("  GPU layer, scores loaded")
    y, io, x = _run(cfg, inp, out["logits"])
    assert np.array_equal(io["topk_idx"].cpu().numpy(), out["topk_idx"])
    assert np.array_equal(io["demand"].cpu().numpy(), out["demand"])
    assert np.array_equal(io["counts"].cpu().numpy(), out["counts"])
    assert np.array_equal(io["offsets"].cpu().numpy(), out["offsets"])
    R = int(out["offsets"][-1])
    row_of = io["row_of"].cpu().numpy()
    src_of = io["src_of"].cpu().numpy()[:R]
    # the keep rule on the GPU's own gates, exactly; differences from the
    # oracle's own keep only at gate near-ties
    flips = check_keep(cfg, io, out)
    log(f"  keep decisions that differ from the oracle's: {len(flips)} of {row_of.size}")
    if cfg.drop != 2:
        assert len(flips) == 0
        assert np.array_equal(row_of, out["row_of"])
        assert np.array_equal(src_of, out["src_of"])
    # x_perm rows are bitwise copies of their source rows (sample of rows)
    rng = np.random.default_rng(5)
    rows = rng.choice(R, size=min(R, 64), replace=False)
    src = (io["z"] if cfg.latent_proj else x).float().cpu().numpy()
    xp = io["x_perm"].float().cpu().numpy()
    idx = io["topk_idx"].cpu().numpy().reshape(-1)
    K = cfg.k_total
    for r in rows:
        a = int(src_of[r])
        h = int(idx[a]) // cfg.e_per_head
        assert np.array_equal(xp[r], src[a // K, h * cfg.d_head:(h + 1) * cfg.d_head])
    if cfg.latent_proj:
        zg = f64(io["z"][torch.from_numpy(toks).cuda()])
        assert np.max(np.abs(zg - out["z"][toks])) <= 2e-2 * np.max(np.abs(out["z"][toks]))
    got = f64(y)[toks]
    ref = out["y"]
    # a sampled token with a near-tie keep flip has another correct output; none is expected
    ok = np.all((row_of[toks] >= 0) == (out["row_of"][toks] >= 0), axis=1)
    assert ok.sum() >= len(toks) - 1
    err = np.max(np.abs(got[ok] - ref[ok]))
    log(f"  sampled rows: max err {err:.3g}, rel {err / np.max(np.abs(ref)):.3g}")
    assert err <= tol(cfg) * np.max(np.abs(ref))


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fullsize_free_running_routing(cfg):
    """The GPU computes its own scores: within 1e-5*max|l| of the oracle's on the same router input."""
    log(f"full-size free-running {cfg.name}")
    inp = cached_inputs(cfg)
    y, io, x = _run(cfg, inp, None)
    if cfg.latent_proj:
        # the router input is the GPU's own bf16 latent: score it with the oracle
        zin = io["z"].float().cpu().numpy().astype(np.float64)
    else:
        zin = oracle.decode(inp.x)
    ref = oracle.route(cfg, zin, inp.w_router, inp.bias)
    l = io["logits"].cpu().numpy().astype(np.float64)
    err = np.max(np.abs(l - ref["logits"]))
    lmax = np.max(np.abs(ref["logits"]))
    got = io["topk_idx"].cpu().numpy()
    diff = np.nonzero(np.any(got != ref["topk_idx"], axis=1))[0]
    margin = routing_margin(cfg, ref["logits"])
    log(f"  max|dl| {err:.3g} (max|l| {lmax:.3g}); tokens routed differently: {len(diff)}")
    assert err <= 1e-5 * lmax
    assert np.all(margin[diff] <= 4 * err), "routing differs at a token that is not a near-tie"


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fullsize_gather_equals_xperm_path(cfg):
    """Without x_perm the expert FFN gathers its rows inside the GEMM: the layer
    output is bitwise that of the copy path (the path the benchmark times)."""
    log(f"full-size gather vs x_perm {cfg.name}")
    inp = cached_inputs(cfg)
    y1, io1, _ = _run(cfg, inp, None, with_xperm=True)
    y2, io2, _ = _run(cfg, inp, None, with_xperm=False)
    for k in ("topk_idx", "offsets", "row_of"):
        assert torch.equal(io1[k], io2[k])
    R = int(io1["offsets"][-1].item())
    assert torch.equal(io1["src_of"][:R], io2["src_of"][:R])  # rows past R are not written
    b = (lambda t: t.view(torch.int16)) if y1.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(b(y1), b(y2))
