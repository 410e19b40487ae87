"""CPU oracle for the MoE layer backward -- TEST INFRASTRUCTURE ONLY.

Only the tests may import this module; the library never does.

What it computes: the gradients of
    L = sum_t <dy_t, y_t> + lam * l_aux
with respect to the layer input x and every weight, for the forward of
moe_oracle.forward with its discrete decisions (the top-k choice of every
token and the keep rule) held fixed: selection and truncation are piecewise
constant, so their derivative is zero almost everywhere and the gradient
flows through the gate values, the experts and the router probabilities.
Float64 throughout; derived by the chain rule from the definitions that
moe_oracle cites:

  y_t   = [x_t] + [s_t] + sum_{kept j} g_{t,j} F_{e_j}(x_t)       ([MoE-evo] "DeepSeekMoE" items 1-2,
                                                                   "GShard" item 3)
  F_e(v) = W2 h,  h = SiLU(W1 v) * (W3 v)   or  h = max(0, W1 v)   ([EP] "MoE 模型的参数量分析";
                                                                   [MoE-evo] "GShard" item 3)
  g_{t,j} = p_{t,e_j}  (or p_{t,e_j} / sum_{j'} p_{t,e_j'})        ([MoE-evo] "DeepSeekMoE" item 1)
  p_t   = softmax(l_t),  l_t = W_r x_t + b                          ([MoE-evo] "Adaptive Mixtures of
                                                                   Local Experts", gating equation)
  l_aux = sum_e m_e c_e / S,  m_e = (1/S) sum_t p_{t,e}            ([MoE-evo] "GShard" item 1)

Backward, per kept assignment (t, j) on expert e (v = x_t):
  dg_{t,j} = <dy_t, F_e(v)>,   dF = g_{t,j} dy_t
  dW2_e += dF h^T,  dh = W2^T dF
  SwiGLU: da1 = dh * (W3 v) * SiLU'(W1 v),  da3 = dh * SiLU(W1 v)
  ReLU:   da1 = dh * [W1 v > 0]
  dW1_e += da1 v^T,  dW3_e += da3 v^T,  dx_t += W1^T da1 + W3^T da3
Router:
  dp_{t,e_j} = dg_{t,j}                     (no renormalisation)
  dp_{t,e_j} = (dg_{t,j} - sum_j' dg_{t,j'} g_{t,j'}) / P_t,  P_t = sum_j' p_{t,e_j'}   (renormalised)
  dp_{t,e} += lam * c_e / S^2               (aux loss, every e)
  dl_{t,e} = p_{t,e} (dp_{t,e} - sum_e' p_{t,e'} dp_{t,e'})         (softmax Jacobian)
  dW_r += dl^T x,  db += sum_t dl_t,  dx_t += W_r^T dl_t
Shared experts and the residual: the same MLP backward with gate 1, and dx_t += dy_t.

Routing variants: with expert choice every token has one slot per expert
(K = E) and the experts' top-C choice is the keep mask; with the balancing
bias b the decisions used b but are held fixed, and a gate that includes b
(g = p + b, optionally renormalised) has the same derivative in p as
without it, up to the renormalising sum, which then runs over p + b.

The backward is defined for one routing head without the latent projections
(the configurations moe_layer_bwd supports).  The probabilities p are those
of the float64 logits (the forward rounds logits to float32 only to take its
decisions); forward_fixed below is that smooth function, which the
finite-difference pins differentiate.
"""
import numpy as np

from .moe_oracle import decode, softmax, silu, RELU, SWIGLU


def _silu_grad(a):
    """d/da SiLU(a) = s(a) (1 + a (1 - s(a))),  s = logistic sigmoid."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def params_of(inp):
    """The float64 parameters of a generated input set, by name."""
    d = lambda a: None if a is None else decode(a)
    sb = getattr(inp, "sel_bias", None)
    return dict(x=d(inp.x), w_router=d(inp.w_router), bias=None if inp.bias is None else np.asarray(inp.bias, np.float64),
                w1=d(inp.w1), w3=d(inp.w3), w2=d(inp.w2), ws1=d(inp.ws1), ws3=d(inp.ws3), ws2=d(inp.ws2),
                sel_bias=None if sb is None else np.asarray(sb, np.float64))


def _gate_values(cfg, P, pc, idx):
    """Gates from the chosen probabilities pc: p (+ b when the bias is in the gate),
    renormalised if asked; also returns the renormalising sum (None without)."""
    g = pc
    if P.get("sel_bias") is not None and getattr(cfg, "sel_bias_gate", 0):
        g = pc + P["sel_bias"][idx.astype(np.int64)]
    if cfg.renorm:
        S = g.sum(axis=-1, keepdims=True)
        return g / S, S
    return g, None


def _check_cfg(cfg):
    if cfg.n_heads != 1 or cfg.latent_proj:
        raise NotImplementedError("the backward oracle covers one routing head without latent projections")


def forward_fixed(cfg, P, topk_idx, kept, lam=0.0, dy=None):
    """The layer output y (float64) with the decisions held fixed, and L = <dy, y> + lam * l_aux.

    topk_idx [T, k] and kept [T*k] are the forward's decisions.
    """
    _check_cfg(cfg)
    x, T, k = P["x"], cfg.T, cfg.k_total
    l = x @ P["w_router"].T
    if P["bias"] is not None:
        l = l + P["bias"]
    p = softmax(l)
    g, _ = _gate_values(cfg, P, np.take_along_axis(p, topk_idx.astype(np.int64), axis=1), topk_idx)
    y = x.copy() if cfg.residual else np.zeros_like(x)
    keep2 = kept.reshape(T, k)
    for t in range(T):
        for j in range(k):
            if not keep2[t, j]:
                continue
            e = int(topk_idx[t, j])
            y[t] += g[t, j] * _ffn(cfg, P, e, x[t:t + 1])[0]
    if cfg.n_shared:
        for i in range(cfg.n_shared):
            y += _shared_ffn(cfg, P, i, x)
    L = None
    if dy is not None:
        S, E = p.shape
        c = np.bincount(topk_idx.reshape(-1), minlength=cfg.n_experts).astype(np.float64)
        aux = float(np.sum(p.sum(axis=0) / S * c / S))
        L = float(np.sum(dy * y)) + lam * aux
    return y, L


def _ffn(cfg, P, e, v):
    w3 = P["w3"][e] if P["w3"] is not None else None
    a1 = v @ P["w1"][e].T
    h = np.maximum(a1, 0.0) if cfg.act == RELU else silu(a1) * (v @ w3.T)
    return h @ P["w2"][e].T


def _shared_slices(cfg, P, i):
    f = cfg.d_ff
    sl = slice(i * f, (i + 1) * f)
    return P["ws1"][sl], (P["ws3"][sl] if P["ws3"] is not None else None), P["ws2"][:, sl]


def _shared_ffn(cfg, P, i, x):
    w1, w3, w2 = _shared_slices(cfg, P, i)
    a1 = x @ w1.T
    h = np.maximum(a1, 0.0) if cfg.act == RELU else silu(a1) * (x @ w3.T)
    return h @ w2.T


def _mlp_backward(act, v, w1, w3, w2, dF):
    """One MLP F = W2 h(v) on the rows of v: returns dv, dW1, dW3, dW2 for upstream dF."""
    a1 = v @ w1.T
    if act == RELU:
        h = np.maximum(a1, 0.0)
        dh = dF @ w2
        da1 = dh * (a1 > 0)
        da3 = None
    else:
        a3 = v @ w3.T
        h = silu(a1) * a3
        dh = dF @ w2
        da1 = dh * a3 * _silu_grad(a1)
        da3 = dh * silu(a1)
    dW2 = dF.T @ h
    dW1 = da1.T @ v
    dv = da1 @ w1
    dW3 = None
    if da3 is not None:
        dW3 = da3.T @ v
        dv = dv + da3 @ w3
    return dv, dW1, dW3, dW2


def backward(cfg, P, topk_idx, kept, dy, lam=0.0):
    """Gradients of L = <dy, y> + lam * l_aux (see the module docstring), float64.

    Returns dict: dx, dw_router, dbias, dw1, dw3, dw2, dws1, dws3, dws2 (None where absent),
    plus the intermediates dg [T, k] (gate gradients) and dl [T, E] (logit gradients).
    """
    _check_cfg(cfg)
    x, T, k, E = P["x"], cfg.T, cfg.k_total, cfg.n_experts
    dy = np.asarray(dy, np.float64)
    l = x @ P["w_router"].T
    if P["bias"] is not None:
        l = l + P["bias"]
    p = softmax(l)
    idx = topk_idx.astype(np.int64)
    pc = np.take_along_axis(p, idx, axis=1)
    g, Psum = _gate_values(cfg, P, pc, idx)
    keep2 = kept.reshape(T, k)

    dx = dy.copy() if cfg.residual else np.zeros_like(x)
    dw1 = np.zeros_like(P["w1"])
    dw2 = np.zeros_like(P["w2"])
    dw3 = np.zeros_like(P["w3"]) if P["w3"] is not None else None
    dg = np.zeros((T, k))
    for e in range(E):
        rows, cols = np.nonzero((idx == e) & keep2)
        if len(rows) == 0:
            continue
        v = x[rows]
        w3 = P["w3"][e] if P["w3"] is not None else None
        F = _ffn(cfg, P, e, v)
        dg[rows, cols] = np.sum(dy[rows] * F, axis=1)
        dF = g[rows, cols][:, None] * dy[rows]
        dv, a, b, c = _mlp_backward(cfg.act, v, P["w1"][e], w3, P["w2"][e], dF)
        np.add.at(dx, rows, dv)
        dw1[e] += a
        dw2[e] += c
        if b is not None:
            dw3[e] += b

    # router: gates -> probabilities -> logits
    dp = np.zeros_like(p)
    if cfg.renorm:
        dpc = (dg - np.sum(dg * g, axis=1, keepdims=True)) / Psum
    else:
        dpc = dg
    np.add.at(dp, (np.arange(T)[:, None].repeat(k, 1), idx), dpc)
    if lam:
        c = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
        dp += lam * c[None, :] / (T * T)
    dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dw_router = dl.T @ x
    dbias = dl.sum(axis=0)
    dx += dl @ P["w_router"]

    dws1 = dws2 = dws3 = None
    if cfg.n_shared:
        dws1, dws2 = np.zeros_like(P["ws1"]), np.zeros_like(P["ws2"])
        dws3 = np.zeros_like(P["ws3"]) if P["ws3"] is not None else None
        f = cfg.d_ff
        for i in range(cfg.n_shared):
            w1, w3, w2 = _shared_slices(cfg, P, i)
            dv, a, b, c = _mlp_backward(cfg.act, x, w1, w3, w2, dy)
            dx += dv
            dws1[i * f:(i + 1) * f] += a
            dws2[:, i * f:(i + 1) * f] += c
            if b is not None:
                dws3[i * f:(i + 1) * f] += b
    return dict(dx=dx, dw_router=dw_router, dbias=dbias, dw1=dw1, dw3=dw3, dw2=dw2,
                dws1=dws1, dws3=dws3, dws2=dws2, dg=dg, dl=dl)


def _gates_and_p(cfg, P, xt, idx_t):
    l = xt @ P["w_router"].T
    if P["bias"] is not None:
        l = l + P["bias"]
    p = softmax(l)
    pc = np.take_along_axis(p, idx_t.astype(np.int64), axis=-1)
    g, S = _gate_values(cfg, P, pc, idx_t)
    return p, (pc if S is None else S), g


def backward_tokens(cfg, P, topk_idx, kept, dy, lam, tokens, demand):
    """dx of the given tokens only: the same chain rule as `backward`, evaluated per
    token (a token's input gradient depends on its own choices, and on the other
    tokens only through the aux loss's demand counts `demand` [E])."""
    _check_cfg(cfg)
    k, T = cfg.k_total, cfg.T
    keep2 = np.asarray(kept).reshape(T, k)
    out = []
    for t in np.asarray(tokens, np.int64):
        xt = P["x"][t:t + 1]
        idx_t = topk_idx[t:t + 1].astype(np.int64)
        p, S, g = _gates_and_p(cfg, P, xt, idx_t)
        dyt = np.asarray(dy[t:t + 1], np.float64)
        dx = dyt.copy() if cfg.residual else np.zeros_like(dyt)
        dg = np.zeros((1, k))
        for j in range(k):
            if not keep2[t, j]:
                continue
            e = int(idx_t[0, j])
            w3 = P["w3"][e] if P["w3"] is not None else None
            dg[0, j] = float(np.sum(dyt * _ffn(cfg, P, e, xt)))
            dv, _, _, _ = _mlp_backward(cfg.act, xt, P["w1"][e], w3, P["w2"][e], g[0, j] * dyt)
            dx += dv
        dp = np.zeros_like(p)
        dpc = (dg - np.sum(dg * g, axis=1, keepdims=True)) / S if cfg.renorm else dg
        np.add.at(dp, (np.zeros(k, np.int64), idx_t[0]), dpc[0])
        if lam:
            dp += lam * np.asarray(demand, np.float64)[None, :] / (T * T)
        dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dx += dl @ P["w_router"]
        for i in range(cfg.n_shared):
            w1, w3, w2 = _shared_slices(cfg, P, i)
            dv, _, _, _ = _mlp_backward(cfg.act, xt, w1, w3, w2, dyt)
            dx += dv
        out.append(dx[0])
    return np.array(out)


def backward_expert(cfg, P, e, topk_idx, kept, dy, hidden=None):
    """dW1, dW3, dW2 of expert e alone: the sums over its kept rows in `backward`.

    `hidden` (index array) restricts them to those hidden units -- rows of dW1
    and dW3, columns of dW2: F = sum_f W2[:, f] h_f, so a unit's weight
    gradients depend on that unit only (and the upstream dF)."""
    _check_cfg(cfg)
    T, k = cfg.T, cfg.k_total
    idx = topk_idx.astype(np.int64)
    rows, cols = np.nonzero((idx == e) & np.asarray(kept).reshape(T, k))
    xv = P["x"][rows]
    _, _, g = _gates_and_p(cfg, P, xv, idx[rows])
    dF = g[np.arange(len(rows)), cols][:, None] * np.asarray(dy, np.float64)[rows]
    hs = slice(None) if hidden is None else np.asarray(hidden, np.int64)
    w3 = P["w3"][e][hs] if P["w3"] is not None else None
    _, dW1, dW3, dW2 = _mlp_backward(cfg.act, xv, P["w1"][e][hs], w3, P["w2"][e][:, hs], dF)
    return dW1, dW3, dW2
