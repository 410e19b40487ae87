"""The layer under HIP graph capture: moe_layer_fwd (and moe_layer_bwd) allocate nothing,
synchronise nothing and clear their counters with kernels, so a captured call replays
correctly.  Each replay runs on a fresh input written into the captured buffer, with
the program's own eager work and synchronisations between replays, and must equal an
eager call on that input bitwise (same kernels, same order, fixed reduction orders).
"""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_router_amd as moe
from moe_inputs import SMALL, SMALL_VARIANTS, bf16_bits_from_f32
from moe_inputs.configs import MoEConfig
from tests.gpu_util import log, dev, weights_dev, cached_inputs, i32, f32, empty_act

pytestmark = pytest.mark.gpu

CFGS = [SMALL[2], SMALL[3], SMALL[4], SMALL_VARIANTS[0], SMALL_VARIANTS[1]]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _io(cfg):
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = max(moe.moe_rows_upper_bound(cfg), 1)
    return dict(logits=f32(T, E), logits_mode=moe.MOE_LOGITS_COMPUTE_STORE, topk_idx=i32(T, K), topk_w=f32(T, K),
                demand=i32(E), counts=i32(E), offsets=i32(E + 1), row_of=i32(T, K), src_of=i32(Rm),
                y_perm=empty_act(cfg, Rm, cfg.d_head), aux_loss=f32(1) if cfg.n_heads == 1 else None,
                seq_loss=f32(T // cfg.seq_len) if cfg.seq_len else None,
                z=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None,
                o=empty_act(cfg, T, cfg.d_latent) if cfg.latent_proj else None)


def _new_x(cfg, seed):
    a = np.random.default_rng([seed, cfg.tag]).standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    return dev(bf16_bits_from_f32(a) if cfg.act_dtype == 1 else a)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_forward_graph_replays_match_eager(cfg):
    log(f"graph forward {cfg.name}")
    inp = cached_inputs(cfg)
    W = weights_dev(cfg, inp)
    ws = moe.workspace(cfg)
    x = _new_x(cfg, 0)
    y = torch.empty_like(x)
    io = _io(cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream
        moe.moe_layer_fwd(cfg, W, x, y, io, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_fwd(cfg, W, x, y, io, ws)
    torch.cuda.synchronize()
    # eager reference buffers, separate from the captured ones
    ws2, io2 = moe.workspace(cfg), _io(cfg)
    for rep in range(3):
        xin = _new_x(cfg, 10 + rep)
        x.copy_(xin)
        g.replay()
        torch.cuda.synchronize()
        # eager work and a synchronisation between replays
        y2 = torch.empty_like(xin)
        moe.moe_layer_fwd(cfg, W, xin, y2, io2, ws2)
        junk = (xin.float() @ xin.float().T).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(_bits(y), _bits(y2)), f"replay {rep}"
        assert torch.equal(io["offsets"], io2["offsets"]), f"replay {rep}"


def test_backward_graph_replays_match_eager():
    cfg = SMALL[2]
    log(f"graph backward {cfg.name}")
    from tests.test_gpu_backward import _transposed, _grads
    inp = cached_inputs(cfg)
    W = weights_dev(cfg, inp)
    x = _new_x(cfg, 0)
    y = torch.empty_like(x)
    io = _io(cfg)
    moe.moe_layer_fwd(cfg, W, x, y, io, moe.workspace(cfg))
    wt = _transposed(cfg, W)
    dy = _new_x(cfg, 1)
    G = _grads(cfg)
    ws = moe.backward_workspace(cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_layer_bwd(cfg, W, wt, x, dy, 0.5, io, G, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_bwd(cfg, W, wt, x, dy, 0.5, io, G, ws)
    torch.cuda.synchronize()
    ws2 = moe.backward_workspace(cfg)
    for rep in range(3):
        d = _new_x(cfg, 20 + rep)
        dy.copy_(d)
        g.replay()
        torch.cuda.synchronize()
        G2 = _grads(cfg)
        moe.moe_layer_bwd(cfg, W, wt, x, d, 0.5, io, G2, ws2)
        torch.cuda.synchronize()
        for k in G:
            if G[k] is not None:
                assert torch.equal(_bits(G[k]), _bits(G2[k])), (rep, k)


def test_forward_backward_with_kept_preactivations_graph():
    """One captured graph holding moe_layer_fwd that keeps the routed pre-activations
    (io.gu) and moe_layer_bwd that reads them: every replay, on a fresh input, equals an
    eager forward + backward on that input bitwise (y, the kept pre-activations and
    every gradient)."""
    from tests.test_gpu_backward import _transposed, _grads
    # bf16 experts on the grouped GEMM, groups of about 1050 rows: 256-row tiles and their tails
    cfg = MoEConfig("graph_gu_tall", T=2100, d_model=320, n_heads=1, d_head=320, n_experts=4, top_k=2,
                    d_ff=128, renorm=1, tag=77)
    log(f"graph forward+backward with kept pre-activations {cfg.name}")
    inp = cached_inputs(cfg)
    W = weights_dev(cfg, inp)
    wt = _transposed(cfg, W)
    Rm = max(moe.moe_rows_upper_bound(cfg), 1)
    m = 2 if cfg.act == 1 else 1

    def state():
        io = _io(cfg)
        io["gu"] = empty_act(cfg, Rm, m * cfg.d_ff)
        return io, moe.workspace(cfg), moe.backward_workspace(cfg), _grads(cfg)

    x, dy = _new_x(cfg, 0), _new_x(cfg, 1)
    y = torch.empty_like(x)
    io, ws, bws, G = state()

    def step(x_, dy_, y_, io_, ws_, bws_, G_):
        moe.moe_layer_fwd(cfg, W, x_, y_, io_, ws_)
        moe.moe_layer_bwd(cfg, W, wt, x_, dy_, 0.5, io_, G_, bws_)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x, dy, y, io, ws, bws, G)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, dy, y, io, ws, bws, G)
    torch.cuda.synchronize()
    io2, ws2, bws2, _ = state()
    for rep in range(3):
        xin, din = _new_x(cfg, 30 + rep), _new_x(cfg, 40 + rep)
        x.copy_(xin)
        dy.copy_(din)
        g.replay()
        torch.cuda.synchronize()
        y2, G2 = torch.empty_like(xin), _grads(cfg)
        step(xin, din, y2, io2, ws2, bws2, G2)
        junk = (xin.float() @ xin.float().T).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(_bits(y), _bits(y2)), f"replay {rep}: y"
        R = int(io2["offsets"][-1])
        assert torch.equal(_bits(io["gu"][:R]), _bits(io2["gu"][:R])), f"replay {rep}: gu"
        for k in G:
            if G[k] is not None:
                assert torch.equal(_bits(G[k]), _bits(G2[k])), (rep, k)
