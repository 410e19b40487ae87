"""Helpers for the GPU parity tests: host arrays <-> device tensors, oracle runs."""
import functools
import sys

import numpy as np
import torch

import oracle
from moe_inputs import generate, bf16_bits_from_f32


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    """numpy host array (uint16 = bf16 bits) -> device tensor."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def f64(t):
    """device tensor -> float64 numpy (bf16 decoded exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def act_round(cfg, a64):
    """Round float64 values to the layer's activation storage (bf16 bits or float32)."""
    if cfg.act_dtype == 1:
        return bf16_bits_from_f32(np.asarray(a64, np.float32))
    return np.asarray(a64, np.float32)


def empty_act(cfg, *shape):
    return torch.empty(*shape, dtype=torch.bfloat16 if cfg.act_dtype == 1 else torch.float32, device="cuda")


def i32(*shape):
    return torch.full(shape, -7, dtype=torch.int32, device="cuda")


def f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


@functools.lru_cache(maxsize=8)
def cached_inputs(cfg):
    return generate(cfg)


def tol(cfg):
    """max-abs-error bound relative to max|ref|: 1e-4 for float32 layers, 2e-2 for bf16."""
    return 1e-4 if cfg.act_dtype == 0 else 2e-2


def weights_dev(cfg, inp):
    return dict(w_router=dev(inp.w_router), router_bias=dev(inp.bias), w1=dev(inp.w1), w3=dev(inp.w3),
                w2=dev(inp.w2), ws1=dev(inp.ws1), ws3=dev(inp.ws3), ws2=dev(inp.ws2), w_in=dev(inp.w_in),
                w_out=dev(inp.w_out), sel_bias=dev(getattr(inp, "sel_bias", None)))


def routing_margin(cfg, l32):
    """Per token, the smallest gap between scores that decides its choices (per head), on the oracle's
    scores: the chosen experts' order and the gap to the best unchosen one, within the groups the token
    keeps when routing is group-limited, and the gap between the last kept and the best dropped group."""
    T, H, Eh, k = cfg.T, cfg.n_heads, cfg.e_per_head, cfg.top_k
    gap = np.full(T, np.inf)
    for h in range(H):
        lh = l32[:, h * Eh:(h + 1) * Eh].astype(np.float64)
        if cfg.n_groups:
            gs = lh.reshape(T, cfg.n_groups, -1).max(axis=2)
            g = np.sort(gs, axis=1)[:, ::-1]
            if cfg.topk_groups < cfg.n_groups:
                gap = np.minimum(gap, g[:, cfg.topk_groups - 1] - g[:, cfg.topk_groups])
            keep = np.argsort(-gs, axis=1, kind="stable")[:, :cfg.topk_groups]
            allowed = np.zeros((T, cfg.n_groups), bool)
            allowed[np.arange(T)[:, None], keep] = True
            lh = np.where(np.repeat(allowed, Eh // cfg.n_groups, axis=1), lh, -np.inf)
        s = np.sort(lh, axis=1)[:, ::-1]
        if k < Eh and np.all(np.isfinite(s[:, k])):
            gap = np.minimum(gap, s[:, k - 1] - s[:, k])
        elif k < Eh:
            fin = np.isfinite(s[:, k])
            gap[fin] = np.minimum(gap[fin], (s[:, k - 1] - s[:, k])[fin])
        if k > 1:
            gap = np.minimum(gap, np.min(s[:, :k - 1] - s[:, 1:k], axis=1))
    return gap


def check_keep(cfg, io, out, near_ties=True):
    """The GPU's keep rule and permutation against the oracle's.

    (1) The oracle's keep rule applied to the GPU's own routing and float32
        gates gives exactly the GPU's demand, counts, offsets, row_of and
        src_of: the kernels implement the rule bit for bit.
    (2) Where the GPU's kept set differs from the oracle's own (the two sides'
        gates can differ in the last bits), the assignment's oracle gate lies
        within 4 float32 ulp of its expert's keep threshold, the keep-th
        largest oracle gate of that expert: a near-tie, not a rule error.
    near_ties=False: (1) only (the routing itself may differ from the oracle's).
    Returns the flat indices of the assignments whose kept state differs."""
    idx = io["topk_idx"].cpu().numpy()
    w32 = io["topk_w"].cpu().numpy().astype(np.float32)
    own = oracle.keep(cfg, idx, w32)
    for k in ("demand", "counts", "offsets"):
        assert np.array_equal(io[k].cpu().numpy(), own[k]), k
    R = int(own["offsets"][-1])
    row_of = io["row_of"].cpu().numpy()
    assert np.array_equal(row_of, own["row_of"])
    assert np.array_equal(io["src_of"].cpu().numpy()[:R], own["src_of"])
    if not near_ties:
        return np.zeros(0, np.int64)
    diff = np.nonzero((row_of.reshape(-1) >= 0) != (out["row_of"].reshape(-1) >= 0))[0]
    if len(diff):
        e_flat = np.asarray(out["topk_idx"]).reshape(-1)
        ow = np.asarray(out["topk_w32"], np.float32).reshape(-1)
        for a in diff:
            e = e_flat[a]
            gates = np.sort(ow[e_flat == e])[::-1]
            keep = int(out["counts"][e])
            thr = gates[keep - 1] if keep > 0 else gates[0]
            assert abs(float(ow[a]) - float(thr)) <= 4 * float(np.spacing(np.float32(thr))), \
                f"assignment {a} (expert {e}) kept differently away from a gate near-tie"
    return diff


def relu_tie_allowance(cfg, P, topk_idx, kept, dy):
    """Element-wise bounds on how far a ReLU layer's gradients may lie from the backward
    oracle's because of the ReLU mask alone.

    The mask [a > 0] of a pre-activation a = W1 v is a decision taken in floating point,
    like the top-k choice: where the oracle's a lies within what the GPU's own a may
    differ from it (float32 sums; with the latent projections also the expert input
    z = x W_in^T, which the layer stores in its activation type and the experts read
    from there), the GPU may take the other side, and its gradients then differ by that
    element's whole term.  Returns (bounds, n) with bounds = {"dx", "dw1", "dw_in" and, with
    shared experts, "dws1"} (the shared experts' masks likewise): the
    sum of those terms' magnitudes over the near-zero elements (zero elsewhere), and n,
    the number of such elements.  Zero bounds for SwiGLU layers (a smooth activation).
    """
    import oracle.moe_backward as OB
    T, E, Eh, dh = cfg.T, cfg.n_experts, cfg.e_per_head, cfg.d_head
    x = P["x"]
    zero = dict(dx=np.zeros_like(x), dw1=np.zeros_like(P["w1"]),
                dw_in=np.zeros_like(P["w_in"]) if cfg.latent_proj else None)
    if cfg.act != 0:
        return zero, 0
    u = OB._u(cfg, P)
    # |what the GPU's a may differ by| <= rel * sum_k |W1 v| (+ z's own rounding and sums)
    rel_z = 2.0 ** -8 if cfg.act_dtype == 1 else 1e-5
    su = np.abs(x) @ np.abs(P["w_in"]).T if cfg.latent_proj else None
    idx = np.asarray(topk_idx, np.int64)
    K = idx.shape[1]
    keep2 = np.asarray(kept).reshape(T, K)
    pc = np.take_along_axis(OB._probs(cfg, P, u), idx, axis=1)
    g, _ = OB._gate_values(cfg, P, pc, idx)
    do = np.asarray(dy, np.float64) @ P["w_out"] if cfg.latent_proj else np.asarray(dy, np.float64)
    b_du = np.zeros((T, cfg.n_heads * dh))
    b_dw1 = np.zeros_like(P["w1"])
    n = 0
    for e in range(E):
        rows, cols = np.nonzero((idx == e) & keep2)
        if len(rows) == 0:
            continue
        hs = slice((e // Eh) * dh, (e // Eh + 1) * dh)
        v, W1 = u[rows, hs], P["w1"][e]
        a = v @ W1.T
        reach = 1e-5 * (np.abs(v) @ np.abs(W1).T)
        if cfg.latent_proj:
            reach += (rel_z * np.abs(v) + 1e-5 * su[rows, hs]) @ np.abs(W1).T
        near = np.abs(a) <= reach
        n += int(near.sum())
        dhid = (g[rows, cols][:, None] * do[rows, hs]) @ P["w2"][e]
        c = np.where(near, np.abs(dhid), 0.0)
        b_dw1[e] += c.T @ np.abs(v)
        np.add.at(b_du, (rows[:, None], np.arange(hs.start, hs.stop)[None, :]), c @ np.abs(W1))
    if cfg.latent_proj:
        return dict(dx=b_du @ np.abs(P["w_in"]), dw1=b_dw1, dw_in=b_du.T @ np.abs(x)), n
    # shared experts (one head, no projections): input x, gate 1, upstream dy
    b_dws1 = np.zeros_like(P["ws1"]) if cfg.n_shared else None
    f = cfg.d_ff
    for i in range(cfg.n_shared):
        w1, _, w2 = OB._shared_slices(cfg, P, i)
        a = x @ w1.T
        near = np.abs(a) <= 1e-5 * (np.abs(x) @ np.abs(w1).T)
        n += int(near.sum())
        c = np.where(near, np.abs(np.asarray(dy, np.float64) @ w2), 0.0)
        b_du += c @ np.abs(w1)
        b_dws1[i * f:(i + 1) * f] += c.T @ np.abs(x)
    return dict(dx=b_du, dw1=b_dw1, dw_in=None, dws1=b_dws1), n
