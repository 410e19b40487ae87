"""GPU: the checked mode for caller-supplied routing (moe_check_topk).

The routing moe_route writes is valid (status 0) for plain, group-limited,
multi-head and expert-choice layers; planted mistakes are each counted: an
expert id below 0, one at E, one from another head's range, and a repeat of
an earlier slot of the same token and head (the top-K selector names K
distinct experts: "MoE技术演进", "Adaptive Mixtures of Local Experts"; per head:
"多头 LatentMoE 与 Head Parallel", 方法论 item 2).  The check only reads the indices.
"""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_router_amd as moe
from moe_inputs import SMALL, SMALL_VARIANTS
from tests.gpu_util import log, dev, cached_inputs

pytestmark = pytest.mark.gpu

CFGS = [SMALL[1], SMALL[3], SMALL[4], SMALL_VARIANTS[3]]  # top-2, group-limited, multi-head, expert choice


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _route(cfg):
    inp = cached_inputs(cfg)
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    if cfg.latent_proj:
        x = torch.randn(T, cfg.d_latent, generator=torch.Generator().manual_seed(5)).to(
            torch.bfloat16 if cfg.act_dtype == 1 else torch.float32).cuda()
    else:
        x = dev(inp.x)
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    gw = torch.empty(T, K, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, x, dev(inp.w_router), dev(inp.bias), None, moe.MOE_LOGITS_COMPUTE, idx, gw, None,
                  moe.workspace(cfg))
    return idx


def _status(cfg, idx):
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_check_topk(cfg, idx, st)
    torch.cuda.synchronize()
    return int(st.item())


@pytest.mark.parametrize("cfg", CFGS, ids=[c.name for c in CFGS])
def test_check_topk(cfg):
    log(f"check_topk {cfg.name}")
    idx = _route(cfg)
    assert _status(cfg, idx) == 0
    T, K, E, H, k = cfg.T, cfg.k_total, cfg.n_experts, cfg.n_heads, cfg.top_k
    bad = idx.cpu().numpy().copy()
    planted = 0
    bad[0, 0] = -1
    planted += 1
    bad[1, K - 1] = E
    planted += 1
    if cfg.route_mode == 1:  # expert choice: slot j must be expert j
        bad[2, 1] = 0
        planted += 1
    else:
        if H > 1:  # an expert of head 1 in a slot of head 0
            bad[2, 0] = cfg.e_per_head + 1
            planted += 1
        if k > 1:  # a repeat of slot 0 (counted once: the later slot)
            bad[3, 1] = bad[3, 0]
            planted += 1
    assert _status(cfg, torch.from_numpy(bad).cuda()) == planted
