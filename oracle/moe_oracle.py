"""CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The library (the C-ABI `libmoe.so` and its Python
binding) never does, and this module imports nothing from the library.

What it computes: the per-token definition of a mixture-of-experts layer,
written out step by step in numpy float64, from inputs decoded exactly from
their bf16/fp32 storage.  Where a floating-point value decides an integer
(which experts a token picks, which assignments survive the affinity keep
rule), the decision is taken on float32 values, the precision the GPU kernels
compute those values in; the float64 values are rounded to float32 once for
that purpose.

Sources (page titles as published; sections as headed on each page):
  [MoE-evo]   "MoE技术演进" (xfliu1998.github.io) -- sections "Adaptive Mixtures
              of Local Experts", "GShard", "DeepSeekMoE", "DeepSeek-V2", "DeepSeek-V3".
  [EP]        "大语言模型并行策略（七）：专家并行" (blog-9y3.pages.dev) -- sections
              "Mixture of Experts (MoE)" and "MoE 模型的参数量分析".
  [LatentMoE] "多头 LatentMoE 与 Head Parallel" (euno.news summary of arXiv
              2602.04870) -- section "方法论" items 1-2.
  [LocMoE+]   jiqizhixin.com article on LocMoE+ -- router-taxonomy paragraph
              (token-choice router with per-expert truncation at capacity C;
              expert-choice router: every expert picks its top-C tokens).

Readings of points the pages leave open are listed in the design doc
("Readings"); the ones used here are restated at the function that uses them.
"""
import numpy as np

RELU, SWIGLU = 0, 1
DROP_NONE, DROP_CAPACITY, DROP_AFFINITY = 0, 1, 2
ROUTE_TOKEN_CHOICE, ROUTE_EXPERT_CHOICE = 0, 1


# --------------------------------------------------------------------------- storage
def decode(a):
    """bf16 bits (uint16) or float32 -> float64, exactly."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- routing
def router_logits(xr, w_r, bias=None):
    """Unnormalised gate scores g_e(x) = <x, W_r[e]> (+ b_e).

    The gating network's scores that the softmax normalises
    ([MoE-evo] "Adaptive Mixtures of Local Experts", gating equation; [EP]
    "Mixture of Experts (MoE)": the router is a linear layer followed by a
    softmax).  The per-expert additive bias is the workload's hot-expert
    bias.  Computed in float64, returned as float32 (the decision precision),
    with -0.0 folded to +0.0 so that equal scores compare equal as keys.
    """
    l = xr @ w_r.T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)
    l32 = l.astype(np.float32) + np.float32(0.0)
    if not np.all(np.isfinite(l32)):
        raise ValueError("non-finite router logit")
    return l32


def softmax(l):
    """p_e = exp(g_e) / sum_j exp(g_j)  ([MoE-evo] gating equation), float64.

    The row maximum is subtracted first; in exact arithmetic that leaves p unchanged.
    """
    l = np.asarray(l, np.float64)
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


def select_topk(l32, k, n_groups=0, topk_groups=0):
    """Indices of the k experts with the largest scores, per row.

    Top-K selector over the gate weights ([MoE-evo] "Adaptive Mixtures of Local
    Experts", selector bullet; [EP] "Mixture of Experts (MoE)").  Selection is
    on the logits, which orders experts exactly as the softmax probabilities
    do.  Order: score descending, lower expert index first on ties; the
    returned row lists the chosen experts in that order.

    Group-limited form ([MoE-evo] "DeepSeek-V2" item 3, device-limited routing:
    first choose M devices, then top-K among their experts; here the devices
    are groups of consecutive experts): a group's score is the largest logit
    in it; the `topk_groups` best groups (score descending, lower group index
    on ties) are kept and top-k runs over their experts only.
    """
    l32 = np.asarray(l32, np.float32)
    T, E = l32.shape
    if n_groups:
        gsz = E // n_groups
        gs = l32.reshape(T, n_groups, gsz).max(axis=2)
        gsel = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
        allow = np.zeros((T, n_groups), bool)
        allow[np.arange(T)[:, None], gsel] = True
        l32 = np.where(np.repeat(allow, gsz, axis=1), l32, np.float32(-np.inf))
    return np.argsort(-l32, axis=1, kind="stable")[:, :k].astype(np.int32)


def gates(p, idx, renorm):
    """Gate of each chosen expert: its softmax probability, optionally renormalised.

    g_{i,t} is the gate value of a selected expert ([MoE-evo] "DeepSeekMoE"
    item 1).  Without renormalisation it is the probability itself; with it,
    the chosen gates are divided by their sum (the coarse workload's rule).
    """
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def aux_loss(p, idx):
    """GShard auxiliary loss  l_aux = sum_e m_e * (c_e / S),  m_e = (1/S) sum_s g_{s,e}.

    ([MoE-evo] "GShard" item 1, auxiliary-loss equation.)  g_{s,e} is the
    dense softmax probability, c_e the number of (token, choice) pairs that
    picked expert e before any drop, S the number of tokens.
    """
    S, E = p.shape
    m = p.sum(axis=0) / S
    c = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
    return float(np.sum(m * c / S))


def biased_keys(p, sel_bias):
    """Selection keys s_{i,t} + b_i of the balancing bias, in float32.

    ([MoE-evo] "DeepSeek-V3" item 1: a per-expert bias b_i is added to the
    token-expert affinity s_{i,t} and the top-K of the sums is selected.)
    The affinity is the softmax probability (the pages' gating score).  The
    float64 probability is rounded to float32 once and the bias added in
    float32: the precision the kernel takes this decision in.
    """
    return (np.asarray(p, np.float64).astype(np.float32) + np.asarray(sel_bias, np.float32)) + np.float32(0.0)


def select_topk_keys(keys, k, n_groups=0, topk_groups=0):
    """Top-k by an explicit float32 key (key descending, lower index first on ties).

    The same selector as select_topk, taking its order from `keys` instead of
    the logits; the group score is the largest key in the group.
    """
    return select_topk(keys, k, n_groups, topk_groups)


def biased_gates(p, sel_bias, idx, renorm, bias_in_gate):
    """Gates under the balancing bias ([MoE-evo] "DeepSeek-V3" item 1).

    The printed formula gives a chosen expert the value s_{i,t} + b_i and
    every other expert 0; with bias_in_gate == 0 the gate is s_{i,t} alone
    (the bias only steers selection).  Renormalisation, when asked for,
    divides by the chosen values' sum as for the plain gates.
    """
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if bias_in_gate:
        w = w + np.asarray(sel_bias, np.float64)[idx]
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def sel_bias_update(sel_bias, counts, gamma):
    """One update of the balancing bias ([MoE-evo] "DeepSeek-V3" item 1).

    An overloaded expert's bias falls by gamma, an underloaded one's rises by
    gamma.  Reading: the load is the number of tokens that chose the expert
    in this batch and "overloaded" means above the mean load over the
    experts; an expert exactly at the mean keeps its bias.  The comparison
    c_e * E versus sum(c) is done in integers.
    """
    c = np.asarray(counts, np.int64)
    E = len(c)
    tot = int(c.sum())
    step = np.sign(tot - c * E).astype(np.float32)  # +1 underloaded, -1 overloaded
    return (np.asarray(sel_bias, np.float32) + np.float32(gamma) * step).astype(np.float32)


def seq_balance(p, idx, seq_len):
    """Per-sequence balance statistic  sum_i f_i P_i  ([MoE-evo] "DeepSeek-V3" item 4).

    For each run of seq_len consecutive tokens: f_i is expert i's load
    frequency, the number of the sequence's (token, choice) pairs that chose
    i divided by the sequence length (the same normalisation as GShard's
    c_e / S, item 1), and P_i the mean probability of i over the sequence.
    The complementary loss is alpha times this value (alpha = 0.0001 on the
    page); the caller applies alpha.
    """
    T, E = p.shape
    L = int(seq_len)
    out = np.zeros(T // L, np.float64)
    for s in range(T // L):
        ps = p[s * L:(s + 1) * L]
        c = np.bincount(idx[s * L:(s + 1) * L].reshape(-1), minlength=E).astype(np.float64)
        out[s] = float(np.sum((c / L) * (ps.sum(axis=0) / L)))
    return out


# --------------------------------------------------------------------------- keep rules
def keep_capacity(e_flat, n_experts, C):
    """Token-choice routing truncated at capacity C per expert.

    Each expert accepts at most C assignments; the overflow goes through the
    residual connection ([MoE-evo] "GShard" item 1, capacity bullet; [LocMoE+]
    truncation of each expert's tokens at C).  Priority is first come in flat
    order a = t*K + j (token-major, then choice rank).
    """
    kept = np.zeros(len(e_flat), bool)
    seen = np.zeros(n_experts, np.int64)
    for a, e in enumerate(e_flat.tolist()):
        kept[a] = seen[e] < C
        seen[e] += 1
    return kept


def keep_affinity(e_flat, w32_flat, n_experts, num, den):
    """Per expert, keep the ceil(num/den) share of its assignments with the highest affinity.

    ([MoE-evo] "DeepSeek-V2" item 5: sort by affinity score, keep the top 90 %,
    drop the rest.)  Scope is one expert; the affinity is the assignment's gate
    (float32); ties go to the smaller flat index; the kept count is
    ceil(num * n_e / den) in integer arithmetic.
    """
    kept = np.zeros(len(e_flat), bool)
    for e in range(n_experts):
        members = np.nonzero(e_flat == e)[0].tolist()
        n = len(members)
        keep = (num * n + den - 1) // den
        ranked = sorted(members, key=lambda a: (-float(w32_flat[a]), a))
        kept[ranked[:keep]] = True
    return kept


def keep_expert_choice(e_flat, w32_flat, n_experts, C):
    """Expert-choice routing: every expert keeps its top-C tokens by gate.

    ([LocMoE+] router-taxonomy paragraph: the expert-choice router lets each
    expert select the top-C tokens that suit it.)  Every token offers one
    assignment to every expert (flat index a = t*E + e, gate = p_{t,e}); per
    expert the min(C, T) assignments with the largest float32 gate are kept,
    ties to the smaller flat index (the earlier token).
    """
    kept = np.zeros(len(e_flat), bool)
    for e in range(n_experts):
        members = np.nonzero(e_flat == e)[0].tolist()
        ranked = sorted(members, key=lambda a: (-float(w32_flat[a]), a))
        kept[ranked[:min(C, len(members))]] = True
    return kept


def permutation(e_flat, kept, n_experts):
    """Expert-contiguous order of the kept assignments.

    Rows of expert e occupy [offsets[e], offsets[e+1]) in ascending flat index
    (the per-expert token buffer of [EP] "MoE 中的 all-to-all 通信", without
    padding).  row_of[a] is the row of assignment a or -1 if dropped;
    src_of[r] is the flat assignment stored at row r.
    """
    n = len(e_flat)
    demand = np.bincount(e_flat, minlength=n_experts).astype(np.int64)
    counts = np.zeros(n_experts, np.int64)
    row_of = np.full(n, -1, np.int64)
    for a in range(n):
        if kept[a]:
            counts[e_flat[a]] += 1
    offsets = np.zeros(n_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    src_of = np.zeros(int(offsets[-1]), np.int64)
    for a in range(n):
        if kept[a]:
            e = e_flat[a]
            row_of[a] = fill[e]
            src_of[fill[e]] = a
            fill[e] += 1
    return demand, counts, offsets, row_of, src_of


# --------------------------------------------------------------------------- experts
def silu(a):
    """SiLU(a) = a / (1 + exp(-a))."""
    return a / (1.0 + np.exp(-a))


def expert_ffn(v, w1, w3, w2, act):
    """One expert's FFN on the rows of v, float64.

    ReLU:   W2 . max(0, W1 v)                  ([MoE-evo] "GShard" item 3, FFN equation)
    SwiGLU: W2 . (SiLU(W1 v) * (W3 v))         (three matrices of d_model x d_moe,
                                                [EP] "MoE 模型的参数量分析")
    No biases.
    """
    h1 = v @ w1.T
    if act == RELU:
        h = np.maximum(h1, 0.0)
    else:
        h = silu(h1) * (v @ w3.T)
    return h @ w2.T


# --------------------------------------------------------------------------- layer
def route(cfg, zr, w_router, bias=None, logits=None, sel_bias=None):
    """Routing of every token: logits, probabilities, top-k, gates (+ aux for one head).

    Per head h the router reads the head's slice of its input and softmaxes
    over the head's own fixed partition of E_h experts ([LatentMoE] 方法论
    item 2: each head picks from its pre-assigned partition); global expert id
    = h * E_h + local id.  With one head this is the ordinary router.
    `logits` (float32 [T, E]) replaces the computed scores when given.
    """
    T, H, dh, Eh, k = cfg.T, cfg.n_heads, cfg.d_head, cfg.e_per_head, cfg.top_k
    w_r = decode(w_router)
    l32 = np.empty((T, cfg.n_experts), np.float32)
    if logits is not None:
        l32[...] = np.asarray(logits, np.float32) + np.float32(0.0)
    else:
        for h in range(H):
            b = None if bias is None else bias[h * Eh:(h + 1) * Eh]
            l32[:, h * Eh:(h + 1) * Eh] = router_logits(
                zr[:, h * dh:(h + 1) * dh], w_r[h * Eh:(h + 1) * Eh], b)
    p = np.empty((T, cfg.n_experts), np.float64)
    for h in range(H):
        sl = slice(h * Eh, (h + 1) * Eh)
        p[:, sl] = softmax(l32[:, sl])
    if getattr(cfg, "route_mode", ROUTE_TOKEN_CHOICE) == ROUTE_EXPERT_CHOICE:
        # expert choice (one head): every token offers every expert; the
        # experts' own top-C choice is the keep rule
        E = cfg.n_experts
        idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
        w = p.copy()
    else:
        idx = np.empty((T, H * k), np.int32)
        for h in range(H):
            sl = slice(h * Eh, (h + 1) * Eh)
            if sel_bias is None:
                idx[:, h * k:(h + 1) * k] = h * Eh + select_topk(l32[:, sl], k, cfg.n_groups, cfg.topk_groups)
            else:
                keys = biased_keys(p[:, sl], sel_bias[sl])
                idx[:, h * k:(h + 1) * k] = h * Eh + select_topk_keys(keys, k, cfg.n_groups, cfg.topk_groups)
        w = np.empty((T, H * k), np.float64)
        for h in range(H):
            ih = idx[:, h * k:(h + 1) * k]
            if sel_bias is None:
                w[:, h * k:(h + 1) * k] = gates(p, ih, cfg.renorm)
            else:
                w[:, h * k:(h + 1) * k] = biased_gates(p, sel_bias, ih, cfg.renorm, cfg.sel_bias_gate)
    aux = aux_loss(p, idx) if H == 1 else None
    seq = seq_balance(p, idx, cfg.seq_len) if getattr(cfg, "seq_len", 0) else None
    return dict(logits=l32, p=p, topk_idx=idx, topk_w=w, topk_w32=w.astype(np.float32), aux=aux, seq=seq)


def keep(cfg, topk_idx, topk_w32):
    """Keep rule over the flat assignments a = t*(H*k) + j."""
    e_flat = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    if getattr(cfg, "route_mode", ROUTE_TOKEN_CHOICE) == ROUTE_EXPERT_CHOICE:
        kept = keep_expert_choice(e_flat, np.asarray(topk_w32, np.float32).reshape(-1), cfg.n_experts,
                                  cfg.capacity)
    elif cfg.drop == DROP_NONE:
        # no token dropping ([MoE-evo] "DeepSeek-V3" item 5)
        kept = np.ones(len(e_flat), bool)
    elif cfg.drop == DROP_CAPACITY:
        kept = keep_capacity(e_flat, cfg.n_experts, cfg.capacity)
    else:
        kept = keep_affinity(e_flat, np.asarray(topk_w32, np.float32).reshape(-1),
                             cfg.n_experts, cfg.keep_num, cfg.keep_den)
    demand, counts, offsets, row_of, src_of = permutation(e_flat, kept, cfg.n_experts)
    return dict(kept=kept, demand=demand, counts=counts, offsets=offsets,
                row_of=row_of.reshape(topk_idx.shape), src_of=src_of)


def forward(cfg, inp, logits=None, tokens=None, want_xperm=False):
    """The layer forward for the tokens in `tokens` (default: all), float64.

    h_t = sum_{shared i} FFN_i(u_t) + sum_{kept (t,e)} g_{e,t} FFN_e(u_t) + u_t
    ([MoE-evo] "DeepSeekMoE" item 2, shared-expert equation; item 1 for the
    routed sum with residual; "GShard" item 3 for the gate-weighted sum).
    Shared experts are ungated and never dropped.  A dropped assignment adds
    nothing and its gate is not redistributed (overflow passes through the
    residual, [MoE-evo] "GShard" item 1).

    Multi-head latent form ([LatentMoE] 方法论 items 1-2): z = x W_in^T; head h
    routes on z's h-th slice within its own partition; its experts run on
    that slice; o_{t,h} = sum_j g FFN(z_{t,h}); y = o W_out^T + x.

    Routing and the keep rule always cover all T tokens (capacity and the
    affinity rule couple tokens); the expert outputs are evaluated for
    `tokens` only.
    """
    T, H, dh, E = cfg.T, cfg.n_heads, cfg.d_head, cfg.n_experts
    k = E if getattr(cfg, "route_mode", ROUTE_TOKEN_CHOICE) == ROUTE_EXPERT_CHOICE else cfg.top_k
    K = H * k
    x = decode(inp.x)
    z = x @ decode(inp.w_in).T if cfg.latent_proj else x
    r = route(cfg, z, inp.w_router, inp.bias, logits, getattr(inp, "sel_bias", None))
    kp = keep(cfg, r["topk_idx"], r["topk_w32"])
    out = dict(r, **kp, z=z if cfg.latent_proj else None)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    n = len(toks)
    dl = H * dh
    routed = np.zeros((n, dl), np.float64)
    w1, w2 = inp.w1, inp.w2
    w3 = inp.w3
    idx, row_of, w = r["topk_idx"], kp["row_of"], r["topk_w"]
    for e in range(E):
        h = e // cfg.e_per_head
        hit = (idx[toks, h * k:(h + 1) * k] == e) & (row_of[toks, h * k:(h + 1) * k] >= 0)
        rows, cols = np.nonzero(hit)
        if len(rows) == 0:
            continue
        cols = cols + h * k
        v = z[toks[rows], h * dh:(h + 1) * dh]
        f = expert_ffn(v, decode(w1[e]), decode(w3[e]) if w3 is not None else None,
                       decode(w2[e]), cfg.act)
        gate = w[toks[rows], cols][:, None]
        np.add.at(routed, (rows[:, None], np.arange(h * dh, (h + 1) * dh)[None, :]), gate * f)
    s = None
    if cfg.n_shared:
        s = np.zeros((n, cfg.d_model), np.float64)
        ws1, ws2 = decode(inp.ws1), decode(inp.ws2)
        ws3 = decode(inp.ws3) if inp.ws3 is not None else None
        f = cfg.d_ff
        for i in range(cfg.n_shared):
            s += expert_ffn(x[toks], ws1[i * f:(i + 1) * f],
                            ws3[i * f:(i + 1) * f] if ws3 is not None else None,
                            ws2[:, i * f:(i + 1) * f], cfg.act)
    if cfg.latent_proj:
        o = routed
        y = o @ decode(inp.w_out).T + x[toks]
        out.update(o=o)
    else:
        y = routed
        if s is not None:
            y = y + s
        if cfg.residual:
            y = y + x[toks]
    out.update(y=y, s=s, tokens=toks)
    if want_xperm:
        src = kp["src_of"]
        t_of = src // K
        e_of = idx.reshape(-1)[src]
        h_of = e_of // cfg.e_per_head
        if cfg.latent_proj or H > 1:
            xp = np.stack([z[t, h * dh:(h + 1) * dh] for t, h in zip(t_of, h_of)]) if len(src) else np.zeros((0, dh))
        else:
            xp = x[t_of]
        out.update(x_perm=xp)
    return out
