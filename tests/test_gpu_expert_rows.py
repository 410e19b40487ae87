"""GPU parity of the expert FFN at hand-picked row counts per expert.

`moe_expert_ffn` takes the expert row ranges (offsets) from the caller, so the
tile edges can be hit directly: experts with 0, 1, 15, 16, 17, 255, 256, 257
and 600 rows, for expert widths that take the fused narrow-expert MLP (64,
128, 256 in bf16) and hidden widths of two to sixteen 32-unit chunks (two:
as many chunks as the three-stage ring keeps in flight), with SwiGLU and
ReLU.  Each expert's rows are checked against the
oracle's FFN ("MoE技术演进", "GShard" item 3; SwiGLU: "大语言模型并行策略（七）：专家并行",
"MoE 模型的参数量分析") within 2e-2 of max|ref|.  Rows past offsets[E] must stay
untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_router_amd as moe
from moe_inputs import MoEConfig, generate, bf16_bits_from_f32
from moe_inputs.configs import ACT_RELU, ACT_SWIGLU, BF16, DROP_NONE
from tests.gpu_util import log, dev, f64, tol

pytestmark = pytest.mark.gpu

ROWS = [0, 1, 15, 16, 17, 255, 256, 257, 600]

CASES = [  # (d_e, d_ff, activation): d_ff is a multiple of 64, two or more 32-unit chunks
    (256, 512, ACT_SWIGLU),
    (256, 64, ACT_SWIGLU),
    (256, 128, ACT_RELU),
    (128, 192, ACT_SWIGLU),
    (128, 128, ACT_RELU),
    (64, 64, ACT_SWIGLU),
    (64, 192, ACT_RELU),
]


def _cfg(dh, dff, act, i):
    E = len(ROWS)
    R = sum(ROWS)
    T = (R + 8) // 2 + 8  # top-2, no drop: room for R rows and a few past them
    return MoEConfig(f"rows{i}_d{dh}_f{dff}", T=T, d_model=dh, n_heads=1, d_head=dh, n_experts=E, top_k=2,
                     drop=DROP_NONE, d_ff=dff, act=act, act_dtype=BF16, router_dtype=BF16, tag=300 + i)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"d{c[0]}_f{c[1]}_{'swiglu' if c[2] else 'relu'}"
                                                       for c in CASES])
def test_expert_ffn_row_edges(i):
    dh, dff, act = CASES[i]
    cfg = _cfg(dh, dff, act, i)
    log(f"expert_ffn rows {ROWS} d_e={dh} d_ff={dff} act={act}")
    inp = generate(cfg)
    offs = np.concatenate([[0], np.cumsum(ROWS)]).astype(np.int32)
    R = int(offs[-1])
    Rm = moe.moe_rows_upper_bound(cfg)
    assert Rm >= R + 8
    rng = np.random.default_rng([31, i])
    xp_bits = bf16_bits_from_f32(rng.standard_normal((R, dh)).astype(np.float32))
    xp = torch.zeros(Rm, dh, dtype=torch.bfloat16, device="cuda")
    xp[:R] = dev(xp_bits)
    sentinel = -12288.0  # exact in bf16
    yp = torch.full((Rm, dh), sentinel, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(cfg)
    moe.moe_expert_ffn(cfg, xp, dev(offs), dev(inp.w1), dev(inp.w3) if inp.w3 is not None else None, dev(inp.w2),
                       yp, None, None, None, None, None, ws)
    torch.cuda.synchronize()
    got = f64(yp)
    xp64 = oracle.decode(xp_bits)
    for e, n in enumerate(ROWS):
        r0, r1 = offs[e], offs[e + 1]
        if n == 0:
            continue
        ref = oracle.expert_ffn(xp64[r0:r1], oracle.decode(inp.w1[e]),
                                oracle.decode(inp.w3[e]) if inp.w3 is not None else None,
                                oracle.decode(inp.w2[e]), cfg.act)
        err = np.max(np.abs(got[r0:r1] - ref))
        scale = np.max(np.abs(ref))
        assert err <= tol(cfg) * scale, f"expert {e} ({n} rows): max err {err:.3g} vs {scale:.3g}"
    assert np.all(got[R:] == sentinel), "rows past offsets[E] were written"


# Experts tall enough for the grouped GEMM's 256-row tiles (the mean row count
# reaches 1024): each expert's rows are cut where its last 256-row tile would
# hold at most 128 rows, the head going to 256 x 256 tiles and the short tail
# to a second launch.  Tails of 1, 64, 65, 128 and 20 rows; 1153, 1280 and 2047
# rows have none.  d_e = 512 takes the grouped GEMM (not the fused MLP); with
# d_ff = 256 both products' tails run the 128 x 64 deep-ring tile (paired
# gate/up rows, then the plain down product), with d_ff = 4096 the gate/up tail
# runs 128 x 128 tiles.
ROWS_TALL = [1025, 1088, 1089, 1152, 1153, 1280, 2047, 0, 1300]
CASES_TALL = [(512, 256, ACT_SWIGLU), (512, 256, ACT_RELU), (512, 4096, ACT_SWIGLU)]


@pytest.mark.parametrize("i", range(len(CASES_TALL)),
                         ids=[f"d{c[0]}_f{c[1]}_{'swiglu' if c[2] else 'relu'}" for c in CASES_TALL])
def test_grouped_gemm_tail_edges(i):
    dh, dff, act = CASES_TALL[i]
    E = len(ROWS_TALL)
    R = sum(ROWS_TALL)
    T = (R + 8) // 2 + 8
    cfg = MoEConfig(f"tall{i}_d{dh}_f{dff}", T=T, d_model=dh, n_heads=1, d_head=dh, n_experts=E, top_k=2,
                    drop=DROP_NONE, d_ff=dff, act=act, act_dtype=BF16, router_dtype=BF16, tag=320 + i)
    assert moe.moe_rows_upper_bound(cfg) // E >= 1024  # the 256-row tiles
    log(f"grouped gemm rows {ROWS_TALL} d_e={dh} d_ff={dff} act={act}")
    inp = generate(cfg)
    offs = np.concatenate([[0], np.cumsum(ROWS_TALL)]).astype(np.int32)
    Rm = moe.moe_rows_upper_bound(cfg)
    rng = np.random.default_rng([37, i])
    xp_bits = bf16_bits_from_f32(rng.standard_normal((R, dh)).astype(np.float32))
    xp = torch.zeros(Rm, dh, dtype=torch.bfloat16, device="cuda")
    xp[:R] = dev(xp_bits)
    sentinel = -12288.0
    yp = torch.full((Rm, dh), sentinel, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(cfg)
    moe.moe_expert_ffn(cfg, xp, dev(offs), dev(inp.w1), dev(inp.w3) if inp.w3 is not None else None, dev(inp.w2),
                       yp, None, None, None, None, None, ws)
    torch.cuda.synchronize()
    got = f64(yp)
    xp64 = oracle.decode(xp_bits)
    for e, n in enumerate(ROWS_TALL):
        r0, r1 = offs[e], offs[e + 1]
        if n == 0:
            continue
        ref = oracle.expert_ffn(xp64[r0:r1], oracle.decode(inp.w1[e]),
                                oracle.decode(inp.w3[e]) if inp.w3 is not None else None,
                                oracle.decode(inp.w2[e]), cfg.act)
        err = np.max(np.abs(got[r0:r1] - ref))
        scale = np.max(np.abs(ref))
        assert err <= tol(cfg) * scale, f"expert {e} ({n} rows): max err {err:.3g} vs {scale:.3g}"
    assert np.all(got[R:] == sentinel), "rows past offsets[E] were written"
