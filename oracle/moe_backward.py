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
  dp_{t,e} += alpha * c_{s,e} / L^2         (sequence-wise balance term, t in sequence s)
Shared experts and the residual: the same MLP backward with gate 1, and dx_t += dy_t.

Routing variants: with expert choice every token has one slot per expert
(K = E) and the experts' top-C choice is the keep mask; with the balancing
bias b the decisions used b but are held fixed, and a gate that includes b
(g = p + b, optionally renormalised) has the same derivative in p as
without it, up to the renormalising sum, which then runs over p + b.

Several routing heads and the latent projections ([LatentMoE] 方法论 items
1-2): u = x W_in^T (or u = x), head h routes on u's h-th slice within its own
E_h experts (softmax and renormalisation per head) and its experts run on that
slice, o_{t,h} = sum_{j in head h} g_{t,j} F_e(u_{t,h}); y = o W_out^T + x.
Then do = dy W_out, dW_out = dy^T o, the per-head backward above runs with do
in place of dy and u in place of x (giving du), dW_in = du^T x and
dx = dy + du W_in.  The aux loss is defined for one head only.

The probabilities p are those
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
                sel_bias=None if sb is None else np.asarray(sb, np.float64),
                w_in=d(getattr(inp, "w_in", None)), w_out=d(getattr(inp, "w_out", None)))


def _u(cfg, P, x=None):
    """Expert and router input: the latent u = x W_in^T, or x itself."""
    x = P["x"] if x is None else x
    return x @ P["w_in"].T if cfg.latent_proj else x


def _probs(cfg, P, u):
    """p [n, E]: per head h, softmax over its E_h experts of u_h W_r[h]^T (+ b_h)."""
    H, Eh, dh = cfg.n_heads, cfg.e_per_head, cfg.d_head
    p = np.empty((u.shape[0], cfg.n_experts))
    for h in range(H):
        rows = slice(h * Eh, (h + 1) * Eh)
        l = u[:, h * dh:(h + 1) * dh] @ P["w_router"][rows].T
        if P["bias"] is not None:
            l = l + P["bias"][rows]
        p[:, rows] = softmax(l)
    return p


def _kh(cfg):
    """Slots per head (k) and per token (K = H k)."""
    K = cfg.k_total
    return K // cfg.n_heads, K


def _gate_values(cfg, P, pc, idx):
    """Gates from the chosen probabilities pc: p (+ b when the bias is in the gate),
    renormalised if asked; also returns the renormalising sum (None without)."""
    g = pc
    if P.get("sel_bias") is not None and getattr(cfg, "sel_bias_gate", 0):
        g = pc + P["sel_bias"][idx.astype(np.int64)]
    if cfg.renorm:
        # per head: the sum over the head's own k slots
        k, K = _kh(cfg)
        n = g.shape[0]
        S = np.repeat(g.reshape(n, K // k, k).sum(axis=2), k, axis=1)
        return g / S, S
    return g, None


def _check_cfg(cfg, lam=0.0):
    if lam and cfg.n_heads != 1:
        raise ValueError("the aux loss is defined for one routing head")


def routed_o(cfg, P, topk_idx, kept, u=None):
    """o [T, H*d_head]: each head's gate-weighted sum of its kept experts on its slice of u."""
    u = _u(cfg, P) if u is None else u
    T, dh, Eh = cfg.T, cfg.d_head, cfg.e_per_head
    k, K = _kh(cfg)
    idx = topk_idx.astype(np.int64)
    g, _ = _gate_values(cfg, P, np.take_along_axis(_probs(cfg, P, u), idx, axis=1), idx)
    keep2 = np.asarray(kept).reshape(T, K)
    o = np.zeros((T, cfg.n_heads * dh))
    for e in range(cfg.n_experts):
        h = e // Eh
        rows, cols = np.nonzero((idx == e) & keep2)
        if len(rows):
            hs = slice(h * dh, (h + 1) * dh)
            o[rows, hs] += g[rows, cols][:, None] * _ffn(cfg, P, e, u[rows, hs])
    return o


def _seq_counts(cfg, topk_idx):
    """c[s][e]: choices of expert e within sequence s (runs of seq_len tokens)."""
    L, E = cfg.seq_len, cfg.n_experts
    idx = np.asarray(topk_idx).astype(np.int64)
    return np.stack([np.bincount(idx[s * L:(s + 1) * L].reshape(-1), minlength=E)
                     for s in range(cfg.T // L)]).astype(np.float64)


def forward_fixed(cfg, P, topk_idx, kept, lam=0.0, dy=None, seq_w=0.0):
    """The layer output y (float64) with the decisions held fixed, and L = <dy, y> + lam * l_aux.

    topk_idx [T, k] and kept [T*k] are the forward's decisions.
    """
    _check_cfg(cfg, lam)
    x, T = P["x"], cfg.T
    u = _u(cfg, P)
    p = _probs(cfg, P, u)
    o = routed_o(cfg, P, topk_idx, kept, u)
    if cfg.latent_proj:
        y = o @ P["w_out"].T + x
    else:
        y = (x.copy() if cfg.residual else np.zeros_like(x)) + o
        for i in range(cfg.n_shared):
            y += _shared_ffn(cfg, P, i, x)
    L = None
    if dy is not None:
        S, E = p.shape
        c = np.bincount(topk_idx.reshape(-1), minlength=cfg.n_experts).astype(np.float64)
        aux = float(np.sum(p.sum(axis=0) / S * c / S))
        L = float(np.sum(dy * y)) + lam * aux
        if seq_w:
            # sequence-wise balance term: sum over sequences of sum_e (c_se / Ls) P_se
            Ls = cfg.seq_len
            cs = _seq_counts(cfg, topk_idx)
            Ps = p.reshape(T // Ls, Ls, -1).sum(axis=1) / Ls
            L += seq_w * float(np.sum(cs / Ls * Ps))
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


def _head_softmax_backward(cfg, p, dp):
    """dl = p (dp - <p, dp>) within each head's experts (softmax Jacobian per head)."""
    Eh = cfg.e_per_head
    dl = np.empty_like(p)
    for h in range(cfg.n_heads):
        rows = slice(h * Eh, (h + 1) * Eh)
        ph, dph = p[:, rows], dp[:, rows]
        dl[:, rows] = ph * (dph - np.sum(ph * dph, axis=1, keepdims=True))
    return dl


def _gate_to_prob_grad(cfg, g, S, dg):
    """dp at the chosen slots from the gate gradients (per-head renormalisation)."""
    if not cfg.renorm:
        return dg
    k, K = _kh(cfg)
    n = dg.shape[0]
    sdg = np.repeat((dg * g).reshape(n, K // k, k).sum(axis=2), k, axis=1)
    return (dg - sdg) / S


def backward(cfg, P, topk_idx, kept, dy, lam=0.0, seq_w=0.0, u=None):
    """Gradients of L = <dy, y> + lam * l_aux [+ seq_w * sum of the per-sequence balance
    terms] (see the module docstring), float64.

    u: the expert and router input to use in place of x W_in^T (a latent layer whose
    z is read at the precision it is stored in); its gradient du passes to W_in and x
    unchanged.  None: u = x W_in^T (or x).

    Returns dict: dx, dw_router, dbias, dw1, dw3, dw2, dws1, dws3, dws2, dw_in, dw_out
    (None where absent), plus the intermediates dg [T, K] (gate gradients), dl [T, E]
    (logit gradients) and du [T, H*d_head] (gradient of the expert input u).
    """
    _check_cfg(cfg, lam)
    x, T, E, Eh, dh = P["x"], cfg.T, cfg.n_experts, cfg.e_per_head, cfg.d_head
    k, K = _kh(cfg)
    dy = np.asarray(dy, np.float64)
    u = _u(cfg, P) if u is None else np.asarray(u, np.float64)
    p = _probs(cfg, P, u)
    idx = topk_idx.astype(np.int64)
    pc = np.take_along_axis(p, idx, axis=1)
    g, S = _gate_values(cfg, P, pc, idx)
    keep2 = np.asarray(kept).reshape(T, K)

    dw_in = dw_out = None
    if cfg.latent_proj:
        o = routed_o(cfg, P, topk_idx, kept, u)
        dw_out = dy.T @ o
        do = dy @ P["w_out"]
    else:
        do = dy
    du = np.zeros((T, cfg.n_heads * dh))
    dw1 = np.zeros_like(P["w1"])
    dw2 = np.zeros_like(P["w2"])
    dw3 = np.zeros_like(P["w3"]) if P["w3"] is not None else None
    dg = np.zeros((T, K))
    for e in range(E):
        rows, cols = np.nonzero((idx == e) & keep2)
        if len(rows) == 0:
            continue
        hs = slice((e // Eh) * dh, (e // Eh + 1) * dh)
        v = u[rows, hs]
        w3 = P["w3"][e] if P["w3"] is not None else None
        F = _ffn(cfg, P, e, v)
        dg[rows, cols] = np.sum(do[rows, hs] * F, axis=1)
        dF = g[rows, cols][:, None] * do[rows, hs]
        dv, a, b, c = _mlp_backward(cfg.act, v, P["w1"][e], w3, P["w2"][e], dF)
        np.add.at(du, (rows[:, None], np.arange(hs.start, hs.stop)[None, :]), dv)
        dw1[e] += a
        dw2[e] += c
        if b is not None:
            dw3[e] += b

    # router: gates -> probabilities -> logits, per head
    dp = np.zeros_like(p)
    np.add.at(dp, (np.arange(T)[:, None].repeat(K, 1), idx), _gate_to_prob_grad(cfg, g, S, dg))
    if lam:
        c = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
        dp += lam * c[None, :] / (T * T)
    if seq_w:
        # d/dp_{t,e} of sum_e (c_se / L) (1/L) sum_{t in s} p_{t,e} = c_se / L^2 for t in s
        Ls = cfg.seq_len
        dp += seq_w * np.repeat(_seq_counts(cfg, topk_idx), Ls, axis=0) / (Ls * Ls)
    dl = _head_softmax_backward(cfg, p, dp)
    dw_router = np.empty_like(P["w_router"])
    for h in range(cfg.n_heads):
        rows = slice(h * Eh, (h + 1) * Eh)
        hs = slice(h * dh, (h + 1) * dh)
        dw_router[rows] = dl[:, rows].T @ u[:, hs]
        du[:, hs] += dl[:, rows] @ P["w_router"][rows]
    dbias = dl.sum(axis=0)

    dws1 = dws2 = dws3 = None
    if cfg.latent_proj:
        dw_in = du.T @ x
        dx = dy + du @ P["w_in"]
    else:
        dx = (dy.copy() if cfg.residual else np.zeros_like(x)) + du
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
                dws1=dws1, dws3=dws3, dws2=dws2, dw_in=dw_in, dw_out=dw_out, dg=dg, dl=dl, du=du)


def backward_tokens(cfg, P, topk_idx, kept, dy, lam, tokens, demand, seq_w=0.0):
    """dx of the given tokens only: the same chain rule as `backward`, evaluated per
    token (a token's input gradient depends on its own choices, and on the other
    tokens only through the aux loss's demand counts `demand` [E])."""
    _check_cfg(cfg, lam)
    T, E, Eh, dh = cfg.T, cfg.n_experts, cfg.e_per_head, cfg.d_head
    k, K = _kh(cfg)
    keep2 = np.asarray(kept).reshape(T, K)
    out = []
    for t in np.asarray(tokens, np.int64):
        xt = P["x"][t:t + 1]
        ut = _u(cfg, P, xt)
        idx_t = topk_idx[t:t + 1].astype(np.int64)
        p = _probs(cfg, P, ut)
        g, S = _gate_values(cfg, P, np.take_along_axis(p, idx_t, axis=1), idx_t)
        dyt = np.asarray(dy[t:t + 1], np.float64)
        dot = dyt @ P["w_out"] if cfg.latent_proj else dyt
        du = np.zeros((1, cfg.n_heads * dh))
        dg = np.zeros((1, K))
        for j in range(K):
            if not keep2[t, j]:
                continue
            e = int(idx_t[0, j])
            hs = slice((e // Eh) * dh, (e // Eh + 1) * dh)
            w3 = P["w3"][e] if P["w3"] is not None else None
            dg[0, j] = float(np.sum(dot[:, hs] * _ffn(cfg, P, e, ut[:, hs])))
            dv, _, _, _ = _mlp_backward(cfg.act, ut[:, hs], P["w1"][e], w3, P["w2"][e], g[0, j] * dot[:, hs])
            du[:, hs] += dv
        dp = np.zeros_like(p)
        np.add.at(dp, (np.zeros(K, np.int64), idx_t[0]), _gate_to_prob_grad(cfg, g, S, dg)[0])
        if lam:
            dp += lam * np.asarray(demand, np.float64)[None, :] / (T * T)
        if seq_w:
            Ls = cfg.seq_len
            dp += seq_w * _seq_counts(cfg, topk_idx)[t // Ls][None, :] / (Ls * Ls)
        dl = _head_softmax_backward(cfg, p, dp)
        for h in range(cfg.n_heads):
            rows = slice(h * Eh, (h + 1) * Eh)
            du[:, h * dh:(h + 1) * dh] += dl[:, rows] @ P["w_router"][rows]
        if cfg.latent_proj:
            dx = dyt + du @ P["w_in"]
        else:
            dx = (dyt.copy() if cfg.residual else np.zeros_like(dyt)) + du
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
    T, Eh, dh = cfg.T, cfg.e_per_head, cfg.d_head
    k, K = _kh(cfg)
    idx = topk_idx.astype(np.int64)
    rows, cols = np.nonzero((idx == e) & np.asarray(kept).reshape(T, K))
    hs = slice((e // Eh) * dh, (e // Eh + 1) * dh)
    xr = P["x"][rows]
    ur = _u(cfg, P, xr)
    p = _probs(cfg, P, ur)
    g, _ = _gate_values(cfg, P, np.take_along_axis(p, idx[rows], axis=1), idx[rows])
    dyr = np.asarray(dy, np.float64)[rows]
    dor = dyr @ P["w_out"] if cfg.latent_proj else dyr
    dF = g[np.arange(len(rows)), cols][:, None] * dor[:, hs]
    hu = slice(None) if hidden is None else np.asarray(hidden, np.int64)
    w3 = P["w3"][e][hu] if P["w3"] is not None else None
    _, dW1, dW3, dW2 = _mlp_backward(cfg.act, ur[:, hs], P["w1"][e][hu], w3, P["w2"][e][:, hu], dF)
    return dW1, dW3, dW2
