"""Dispatch at token counts past the affinity kernel's LDS staging limit, bit-exact against the oracle.

The per-expert selection of the affinity keep rule and of expert choice
stages an expert's keys in LDS when the launch's staging capacity allows it
(capacity min(T, 19968) keys, so 156 KiB of LDS from T = 19968 on) and reads
them from global memory otherwise.  These cases put one hot expert past the
capacity (read from global memory) beside experts that are staged at the
largest capacity, with many equal gates so the tie order (earlier assignment
first) decides the boundary.  Inputs are synthetic top-k lists and gates: the
dispatch takes them as given, so no routing runs here.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_router_amd as moe
from moe_inputs.configs import MoEConfig, DROP_AFFINITY, DROP_CAPACITY, ROUTE_EXPERT_CHOICE, F32
from tests.gpu_util import log, dev, i32

pytestmark = pytest.mark.gpu

STAGE_MAX = (160 * 1024 - 4096) // 8  # keys the kernel stages in LDS at most


def _token_choice(T, E, k, hot, rng):
    """Top-k lists where expert `hot` is the first choice of ~90 % of tokens; quantised gates (ties)."""
    idx = np.empty((T, k), np.int32)
    first = np.where(rng.random(T) < 0.9, hot, rng.integers(0, E, T))
    idx[:, 0] = first
    for j in range(1, k):
        # a distinct expert per slot: shift by a random nonzero offset from the previous choices
        cand = (first + j + rng.integers(0, E - k + 1, T)) % E
        idx[:, j] = cand
    w = (rng.integers(0, 48, (T, k)) / 64.0).astype(np.float32)  # 48 levels incl. 0.0
    return idx, w


def _run(cfg, idx, w, x):
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = moe.moe_rows_upper_bound(cfg)
    ws = moe.workspace(cfg)
    demand, counts, offsets = i32(E), i32(E), i32(E + 1)
    row_of, src_of = i32(T, K), i32(Rm)
    xp = torch.empty(Rm, cfg.d_head, dtype=torch.float32, device="cuda")
    moe.moe_dispatch(cfg, dev(idx), dev(w), dev(x), demand, counts, offsets, row_of, src_of, xp, ws)
    torch.cuda.synchronize()
    return dict(demand=demand.cpu().numpy(), counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                row_of=row_of.cpu().numpy(), src_of=src_of.cpu().numpy(), xp=xp.cpu().numpy())


def _compare(cfg, got, ref, x):
    assert np.array_equal(got["demand"], ref["demand"])
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["row_of"], ref["row_of"])
    R = int(ref["offsets"][-1])
    assert np.array_equal(got["src_of"][:R], ref["src_of"])
    assert np.array_equal(got["xp"][:R], x[ref["src_of"] // cfg.k_total])


@pytest.mark.parametrize("T", [STAGE_MAX + 4032, STAGE_MAX])
def test_affinity_keep_past_lds_staging(T):
    E, k, d = 8, 2, 64
    cfg = MoEConfig(f"aff_large_T{T}", T=T, d_model=d, n_heads=1, d_head=d, n_experts=E, top_k=k,
                    drop=DROP_AFFINITY, keep_num=9, keep_den=10, d_ff=64, act_dtype=F32, router_dtype=F32, tag=90)
    assert moe.moe_check_config(cfg) == 0
    rng = np.random.default_rng([90, T])
    idx, w = _token_choice(T, E, k, hot=3, rng=rng)
    x = rng.standard_normal((T, d)).astype(np.float32)
    log(f"dispatch affinity T={T} E={E} k={k}")
    ref = oracle.keep(cfg, idx, w)
    n_hot = int(ref["demand"][3])
    log(f"  hot expert: {n_hot} assignments (staging capacity {min(T, STAGE_MAX)})")
    if T > STAGE_MAX:
        assert n_hot > STAGE_MAX  # the hot expert takes the global-memory path
    got = _run(cfg, idx, w, x)
    _compare(cfg, got, ref, x)


def test_expert_choice_past_lds_staging():
    T, E, d, C = STAGE_MAX + 1000, 4, 64, 5003
    cfg = MoEConfig("ec_large", T=T, d_model=d, n_heads=1, d_head=d, n_experts=E, top_k=1, drop=DROP_CAPACITY,
                    capacity=C, d_ff=64, act_dtype=F32, router_dtype=F32, route_mode=ROUTE_EXPERT_CHOICE, tag=91)
    assert moe.moe_check_config(cfg) == 0
    rng = np.random.default_rng(91)
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    w = (rng.integers(0, 200, (T, E)) / 256.0).astype(np.float32)  # every key repeated ~100 times
    x = rng.standard_normal((T, d)).astype(np.float32)
    log(f"dispatch expert choice T={T} E={E} C={C}")
    ref = oracle.keep(cfg, idx, w)
    assert np.all(ref["counts"] == C)
    got = _run(cfg, idx, w, x)
    _compare(cfg, got, ref, x)
