"""The layer at the largest supported size: 1 048 000 tokens of width 2048.

moe_check_config bounds every operand the kernels address with 32-bit
element offsets below 2^31 elements; T * d_model = 2 146 304 000 sits just
under that bound (T = 1 048 576 reaches it and is refused).  The forward
runs free (the router computes its scores) with the expert FFN gathering its
rows from x, and is checked against the oracle:
  * scores of sampled tokens (the first and last ones included) within
    1e-5 * max|l| of the oracle's router product;
  * for every token, the choices equal the oracle's selection on the GPU's
    own scores, and the gates equal the oracle's softmax gates within 1e-6;
  * the keep rule and permutation (offsets, row_of, src_of) bit-exact for all
    2 096 000 assignments;
  * y of the sampled tokens within 2e-2 * max|y|.
The backward's transposed buffers would pass 2^31 elements here, so the
backward reports no workspace for this shape.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_router_amd as moe
from moe_inputs import generate
from moe_inputs.configs import MoEConfig
from tests.gpu_util import log, dev, f64, i32, f32, weights_dev

CFG = MoEConfig("max_t1048000_d2048", T=1_048_000, d_model=2048, n_heads=1, d_head=2048, n_experts=8, top_k=2,
                d_ff=64, act=1, drop=0, act_dtype=1, router_dtype=1, residual=1, tag=95)


def test_size_bounds():
    """Host-side: this size is supported, one more row of tokens past 2^31 elements is not."""
    assert moe.moe_check_config(CFG) == moe.MOE_OK
    assert CFG.T * CFG.d_model < 2 ** 31
    assert moe.moe_check_config(CFG.with_(T=1_048_576)) == moe.MOE_ERR_UNSUPPORTED
    assert moe.moe_backward_workspace_bytes(CFG) == 0


@pytest.mark.gpu
def test_layer_at_max_size():
    cfg = CFG
    log(f"max size {cfg.name}: generating inputs")
    inp = generate(cfg, threads=16)
    T, K, E = cfg.T, cfg.k_total, cfg.n_experts
    Rm = moe.moe_rows_upper_bound(cfg)
    io = dict(logits=f32(T, E), logits_mode=moe.MOE_LOGITS_COMPUTE_STORE, topk_idx=i32(T, K), topk_w=f32(T, K),
              demand=i32(E), counts=i32(E), offsets=i32(E + 1), row_of=i32(T, K), src_of=i32(Rm),
              y_perm=torch.empty(Rm, cfg.d_head, dtype=torch.bfloat16, device="cuda"), aux_loss=f32(1))
    x = dev(inp.x)
    y = torch.empty_like(x)
    log("  forward")
    moe.moe_layer_fwd(cfg, weights_dev(cfg, inp), x, y, io, moe.workspace(cfg))
    torch.cuda.synchronize()

    rng = np.random.default_rng(95)
    sample = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T), rng.choice(T, 240, replace=False)]))
    xs = oracle.decode(inp.x[sample])
    l_gpu = io["logits"].cpu().numpy()
    l_ref = oracle.router_logits(xs, oracle.decode(inp.w_router))
    err = np.max(np.abs(l_gpu[sample].astype(np.float64) - l_ref))
    log(f"  sampled scores rel err {err / np.max(np.abs(l_ref)):.3g}")
    assert err <= 1e-5 * np.max(np.abs(l_ref))

    # every token: the oracle's selection and gates on the GPU's own scores
    idx = io["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, oracle.select_topk(l_gpu, cfg.top_k))
    p = oracle.softmax(l_gpu)
    w_ref = oracle.gates(p, idx, cfg.renorm)
    w_gpu = io["topk_w"].cpu().numpy()
    assert np.max(np.abs(w_gpu.astype(np.float64) - w_ref)) <= 1e-6

    log("  keep rule and permutation")
    kp = oracle.keep(cfg, idx, w_gpu)
    assert np.array_equal(io["demand"].cpu().numpy(), kp["demand"])
    assert np.array_equal(io["counts"].cpu().numpy(), kp["counts"])
    assert np.array_equal(io["offsets"].cpu().numpy(), kp["offsets"])
    assert np.array_equal(io["row_of"].cpu().numpy(), kp["row_of"])
    R = int(kp["offsets"][-1])
    assert np.array_equal(io["src_of"].cpu().numpy()[:R], kp["src_of"])

    log("  sampled outputs")
    ys = f64(y[torch.from_numpy(sample).to("cuda")])
    ref = xs.copy()
    w1, w3, w2 = inp.w1, inp.w3, inp.w2
    for i, t in enumerate(sample):
        for j in range(K):
            e = int(idx[t, j])
            f = oracle.expert_ffn(xs[i:i + 1], oracle.decode(w1[e]), oracle.decode(w3[e]), oracle.decode(w2[e]),
                                  cfg.act)
            ref[i] += float(w_gpu[t, j]) * f[0]
    err = np.max(np.abs(ys - ref))
    log(f"  sampled y rel err {err / np.max(np.abs(ref)):.3g}")
    assert err <= 2e-2 * np.max(np.abs(ref))
