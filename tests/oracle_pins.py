"""Checks that pin the CPU oracle to facts outside itself.

Each check raises AssertionError on failure.  They are called by
test_oracle_pins.py directly, and by test_oracle_mutants.py against copies of
the oracle with a planted mistake, to show that each plausible mistake is
caught by at least one of them.

What pins what:
  router scores  a hand-worked two-head example with a bias (tests/golden):
                 per-head slices, the bias added once
  softmax        rows sum to 1; p_i/p_j = exp(l_i - l_j); equal logits -> 1/E;
                 scipy.special.softmax (library routine)
  top-k          brute-force subset enumeration with the total-order invariant
  group-limited  brute force over group subsets, then expert subsets;
                 topk_groups == n_groups reduces to plain top-k
  gates / aux    the hand-worked 4-token example (tests/golden)
  capacity       brute-force O(n^2) rank count; counts == min(n_e, C)
  affinity keep  brute-force dominance count; kept == ceil(9 n / 10)
  permutation    stable argsort (library routine); x_perm rows == source rows
  expert FFN     torch.nn.functional linear/relu/silu in float64 (library)
  combine        dense masked evaluation of every expert on every token
  shared         two shared experts == one with concatenated hidden width
  multi-head     H=1 with identity projections == a top-1 MoE with residual;
                 permuting heads permutes the head slices of o
"""
import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _o():
    import oracle.moe_oracle as m
    return m


# ---------------------------------------------------------------- router scores
def check_router_logits():
    """The hand-worked two-head example of tests/golden/hand_router_logits.json.

    Checked twice: on router_logits itself, one head slice at a time, and
    through route(), which must give head h the columns of its own slice of
    the router input and its own rows of W_r and the bias."""
    O = _o()
    with open(os.path.join(GOLDEN, "hand_router_logits.json")) as f:
        g = json.load(f)
    z = np.array(g["z"], np.float64)
    w = np.array(g["w_router"], np.float32)
    b = np.array(g["bias"], np.float32)
    want = np.array(g["logits"], np.float32)
    H, dh, Eh = g["n_heads"], g["d_head"], g["experts_per_head"]
    for h in range(H):
        got = O.router_logits(z[:, h * dh:(h + 1) * dh], O.decode(w[h * Eh:(h + 1) * Eh]), b[h * Eh:(h + 1) * Eh])
        assert got.dtype == np.float32
        assert np.array_equal(got, want[:, h * Eh:(h + 1) * Eh]), (h, got)
        nob = O.router_logits(z[:, h * dh:(h + 1) * dh], O.decode(w[h * Eh:(h + 1) * Eh]))
        assert np.array_equal(nob, np.array(g["logits_no_bias"], np.float32)[:, h * Eh:(h + 1) * Eh])
    from moe_inputs import MoEConfig
    cfg = MoEConfig("hand_logits", T=2, d_model=H * dh, n_heads=H, d_head=dh, n_experts=H * Eh, top_k=1,
                    d_ff=64, act_dtype=0, router_dtype=0)
    r = O.route(cfg, z, w, b)
    assert np.array_equal(r["logits"], want)
    assert r["topk_idx"].tolist() == g["top1_idx"]
    # -0.0 folds to +0.0: a score that cancels exactly is a +0.0 key
    zero = O.router_logits(np.array([[1.0, -1.0]]), np.array([[1.0, 1.0]]), np.array([-0.0], np.float32))
    assert np.signbit(zero).tolist() == [[False]]


# ---------------------------------------------------------------- softmax
def check_softmax():
    O = _o()
    rng = np.random.default_rng(1)
    l = rng.standard_normal((50, 33)) * 4
    p = O.softmax(l)
    assert np.all(np.abs(p.sum(1) - 1) < 1e-12)
    i, j = 3, 17
    assert np.allclose(p[:, i] / p[:, j], np.exp(l[:, i] - l[:, j]), rtol=1e-12)
    for E in (1, 4, 7, 160):
        q = O.softmax(np.full((2, E), 0.3))
        assert np.all(q == 1.0 / E)
    import scipy.special
    assert np.allclose(p, scipy.special.softmax(l, axis=1), rtol=1e-12, atol=0)


# ---------------------------------------------------------------- top-k
def _beats(l, a, b):
    """(l[a], -a) > (l[b], -b): score descending, lower index first."""
    return l[a] > l[b] or (l[a] == l[b] and a < b)


def _brute_topk(l, k, allowed=None):
    E = len(l)
    cand = range(E) if allowed is None else sorted(allowed)
    good = []
    for S in itertools.combinations(cand, k):
        rest = [e for e in cand if e not in S]
        if all(_beats(l, a, b) for a in S for b in rest):
            good.append(S)
    assert len(good) == 1
    S = list(good[0])
    # listed in order: each beats every later one
    S.sort(key=lambda e: (-l[e], e))
    return S


def _brute_group(l, k, G, gk):
    E = len(l)
    gsz = E // G
    gs = [max(l[g * gsz:(g + 1) * gsz]) for g in range(G)]
    good = []
    for S in itertools.combinations(range(G), gk):
        rest = [g for g in range(G) if g not in S]
        if all(gs[a] > gs[b] or (gs[a] == gs[b] and a < b) for a in S for b in rest):
            good.append(S)
    assert len(good) == 1
    allowed = [e for g in good[0] for e in range(g * gsz, (g + 1) * gsz)]
    return _brute_topk(l, k, allowed)


def check_topk():
    O = _o()
    rng = np.random.default_rng(2)
    for trial in range(40):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        # small integer logits force many ties; include both signed zeros
        l = rng.integers(-2, 3, size=(6, E)).astype(np.float32)
        l[0, 0] = -0.0
        l = l + np.float32(0.0)
        idx = O.select_topk(l, k)
        for t in range(l.shape[0]):
            assert list(idx[t]) == _brute_topk(list(l[t]), k), (l[t], k, idx[t])


def check_topk_groups():
    O = _o()
    rng = np.random.default_rng(3)
    for trial in range(30):
        G = int(rng.integers(1, 5))
        gsz = int(rng.integers(1, 4))
        E = G * gsz
        gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, gk * gsz + 1))
        l = rng.integers(-2, 3, size=(5, E)).astype(np.float32)
        idx = O.select_topk(l, k, G, gk)
        for t in range(l.shape[0]):
            assert list(idx[t]) == _brute_group(list(l[t]), k, G, gk)
        full = O.select_topk(l, k, G, G)
        assert np.array_equal(full, O.select_topk(l, k))


# ---------------------------------------------------------------- hand example
def golden():
    with open(os.path.join(GOLDEN, "hand_4token.json")) as f:
        return json.load(f)


def _hand_cfg(renorm=0, drop=0, C=0):
    from moe_inputs import MoEConfig
    return MoEConfig("hand", T=4, d_model=64, n_heads=1, d_head=64, n_experts=4, top_k=2,
                     renorm=renorm, drop=drop, capacity=C, d_ff=64)


def check_hand_example():
    O = _o()
    g = golden()
    logits = np.log(np.array(g["probs"])).astype(np.float32)
    r = O.route(_hand_cfg(), None, np.zeros((4, 64), np.float32), logits=logits)
    assert r["topk_idx"].tolist() == g["topk_idx"]
    assert np.allclose(r["topk_w"], g["gates"], atol=1e-6)
    assert abs(r["aux"] - g["aux"]) < 1e-6
    m = r["p"].sum(0) / 4
    assert np.allclose(m, g["aux_m"], atol=1e-6)
    assert np.bincount(r["topk_idx"].reshape(-1), minlength=4).tolist() == g["aux_c"]
    rr = O.route(_hand_cfg(renorm=1), None, np.zeros((4, 64), np.float32), logits=logits)
    assert np.allclose(rr["topk_w"], g["gates_renorm"], atol=1e-6)
    kp = O.keep(_hand_cfg(drop=1, C=g["capacity"]), r["topk_idx"], r["topk_w32"])
    assert kp["counts"].tolist() == g["cap_counts"]
    assert kp["offsets"].tolist() == g["cap_offsets"]
    assert kp["src_of"].tolist() == g["cap_src_of"]
    assert kp["row_of"].tolist() == g["cap_row_of"]
    # uniform probabilities with balanced counts: the minimum k/E
    E, k, T = 8, 2, 8
    lu = np.zeros((T, E), np.float32)
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    assert abs(O.aux_loss(O.softmax(lu), idx) - k / E) < 1e-12


# ---------------------------------------------------------------- keep rules
def check_capacity():
    O = _o()
    rng = np.random.default_rng(4)
    for trial in range(20):
        E = int(rng.integers(1, 6))
        n = int(rng.integers(0, 40))
        C = int(rng.integers(0, 8))
        e = rng.integers(0, E, size=n)
        kept = O.keep_capacity(e, E, C)
        brute = [sum(1 for b in range(a) if e[b] == e[a]) < C for a in range(n)]
        assert kept.tolist() == brute
        cnt = np.bincount(e[kept], minlength=E)
        assert np.array_equal(cnt, np.minimum(np.bincount(e, minlength=E), C))
        assert O.keep_capacity(e, E, n).all()


def check_affinity():
    O = _o()
    rng = np.random.default_rng(5)
    for trial in range(20):
        E = int(rng.integers(1, 5))
        n = int(rng.integers(0, 50))
        e = rng.integers(0, E, size=n)
        w = (rng.integers(0, 5, size=n) / 8.0).astype(np.float32)   # ties on purpose
        kept = O.keep_affinity(e, w, E, 9, 10)
        for a in range(n):
            same = [b for b in range(n) if e[b] == e[a]]
            ne = len(same)
            better = sum(1 for b in same if (w[b] > w[a]) or (w[b] == w[a] and b < a))
            assert kept[a] == (better < -(-9 * ne // 10))
        for x in range(E):
            ne = int((e == x).sum())
            assert int(kept[e == x].sum()) == (9 * ne + 9) // 10
        assert O.keep_affinity(e, w, E, 10, 10).all()


def check_permutation():
    O = _o()
    rng = np.random.default_rng(6)
    for trial in range(10):
        E = int(rng.integers(1, 7))
        n = int(rng.integers(0, 60))
        e = rng.integers(0, E, size=n)
        kept = rng.random(n) < 0.7
        demand, counts, offsets, row_of, src_of = O.permutation(e, kept, E)
        ka = np.nonzero(kept)[0]
        ref = ka[np.argsort(e[ka], kind="stable")]
        assert src_of.tolist() == ref.tolist()
        assert np.array_equal(offsets[1:], np.cumsum(np.bincount(e[kept], minlength=E)))
        assert np.array_equal(demand, np.bincount(e, minlength=E))
        assert all(row_of[src_of[r]] == r for r in range(len(src_of)))
        assert np.all(row_of[~kept] == -1)


# ---------------------------------------------------------------- FFN and layer
def _torch_ffn(v, w1, w3, w2, act):
    import torch
    import torch.nn.functional as F
    v, w1, w2 = (torch.from_numpy(np.ascontiguousarray(a)) for a in (v, w1, w2))
    if act == 0:
        h = F.relu(F.linear(v, w1))
    else:
        h = F.silu(F.linear(v, w1)) * F.linear(v, torch.from_numpy(np.ascontiguousarray(w3)))
    return F.linear(h, w2).numpy()


def check_ffn_library():
    O = _o()
    rng = np.random.default_rng(7)
    for act in (0, 1):
        v = rng.standard_normal((9, 16))
        w1 = rng.standard_normal((24, 16))
        w3 = rng.standard_normal((24, 16))
        w2 = rng.standard_normal((16, 24))
        assert np.allclose(O.expert_ffn(v, w1, w3 if act else None, w2, act),
                           _torch_ffn(v, w1, w3, w2, act), rtol=1e-12, atol=1e-12)


def _f32_inputs(cfg):
    from moe_inputs import generate
    return generate(cfg)


def check_dense_special_case():
    """E=1, k=1, renormalised, no drop: the layer is u + FFN(u) (torch)."""
    O = _o()
    from moe_inputs import MoEConfig
    for act in (0, 1):
        cfg = MoEConfig("dense", T=7, d_model=64, n_heads=1, d_head=64, n_experts=1, top_k=1,
                        renorm=1, d_ff=64, act=act, act_dtype=0, router_dtype=0)
        inp = _f32_inputs(cfg)
        y = O.forward(cfg, inp)["y"]
        x = O.decode(inp.x)
        ref = x + _torch_ffn(x, O.decode(inp.w1[0]), O.decode(inp.w3[0]) if act else None,
                             O.decode(inp.w2[0]), act)
        assert np.allclose(y, ref, rtol=1e-10, atol=1e-10)


def check_identical_experts():
    """All experts equal, renormalised gates, no drop: u + FFN(u) whatever the routing."""
    O = _o()
    from moe_inputs import MoEConfig
    cfg = MoEConfig("ident", T=11, d_model=64, n_heads=1, d_head=64, n_experts=5, top_k=3,
                    renorm=1, d_ff=64, act=1, act_dtype=0, router_dtype=0)
    inp = _f32_inputs(cfg)
    for name in ("w1", "w3", "w2"):
        a = getattr(inp, name)
        a[...] = a[0:1]
    y = O.forward(cfg, inp)["y"]
    x = O.decode(inp.x)
    ref = x + _torch_ffn(x, O.decode(inp.w1[0]), O.decode(inp.w3[0]), O.decode(inp.w2[0]), 1)
    assert np.allclose(y, ref, rtol=1e-10, atol=1e-10)


def check_dense_masked():
    """Every expert on every token, times the kept gate mask, summed: same y."""
    O = _o()
    from moe_inputs import SMALL
    for cfg in (SMALL[0], SMALL[2], SMALL[3]):
        cfg = cfg.with_(T=min(cfg.T, 96))
        if cfg.drop == 1:
            cfg = cfg.with_(capacity=max(1, cfg.capacity // 3))
        inp = _f32_inputs(cfg)
        out = O.forward(cfg, inp)
        x = O.decode(inp.x)
        y = x.copy() if cfg.residual else np.zeros_like(x)
        idx, w, kept = out["topk_idx"], out["topk_w"], out["kept"].reshape(out["topk_idx"].shape)
        for e in range(cfg.n_experts):
            gate = ((idx == e) & kept) * w
            f = _torch_ffn(x, O.decode(inp.w1[e]), O.decode(inp.w3[e]) if inp.w3 is not None else None,
                           O.decode(inp.w2[e]), cfg.act)
            y += gate.sum(1, keepdims=True) * f
        if cfg.n_shared:
            fs = cfg.d_ff * cfg.n_shared
            y += _torch_ffn(x, O.decode(inp.ws1).reshape(fs, -1), O.decode(inp.ws3).reshape(fs, -1),
                            O.decode(inp.ws2), cfg.act)
        assert np.allclose(out["y"], y, rtol=1e-9, atol=1e-9)


def check_shared_concat():
    """Two shared experts equal one shared expert with the hidden widths concatenated."""
    O = _o()
    from moe_inputs import SMALL
    cfg = SMALL[2].with_(T=40)
    inp = _f32_inputs(cfg)
    a = O.forward(cfg, inp)["s"]
    x = O.decode(inp.x)
    f = cfg.d_ff
    two = sum(_torch_ffn(x, O.decode(inp.ws1[i * f:(i + 1) * f]), O.decode(inp.ws3[i * f:(i + 1) * f]),
                         O.decode(inp.ws2[:, i * f:(i + 1) * f]), 1) for i in range(2))
    assert np.allclose(a, two, rtol=1e-10, atol=1e-10)


def check_multihead_reductions():
    O = _o()
    from moe_inputs import MoEConfig, generate
    # H = 1, W_in = W_out = I: a top-1 MoE with residual
    cfg_l = MoEConfig("lat1", T=23, d_model=64, n_heads=1, d_head=64, n_experts=6, top_k=1,
                      d_ff=64, latent_proj=1, act_dtype=0, router_dtype=0, zipf_s=1.0)
    inp = generate(cfg_l)
    inp.w_in[...] = np.eye(64, dtype=np.float32)
    inp.w_out[...] = np.eye(64, dtype=np.float32)
    a = O.forward(cfg_l, inp)["y"]
    cfg_p = cfg_l.with_(latent_proj=0)
    b = O.forward(cfg_p, inp)["y"]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # permuting heads permutes o's head slices and leaves y unchanged
    cfg = MoEConfig("lat3", T=17, d_model=64, n_heads=3, d_head=32, n_experts=12, top_k=1,
                    d_ff=32, latent_proj=1, act_dtype=0, router_dtype=0, zipf_s=1.0)
    inp = generate(cfg)
    out = O.forward(cfg, inp)
    perm = [2, 0, 1]
    import copy
    q = copy.deepcopy(inp)
    dh, Eh = 32, 4
    q.w_in[...] = np.concatenate([inp.w_in[h * dh:(h + 1) * dh] for h in perm])
    q.w_out[...] = np.concatenate([inp.w_out[:, h * dh:(h + 1) * dh] for h in perm], axis=1)
    q.w_router[...] = np.concatenate([inp.w_router[h * Eh:(h + 1) * Eh] for h in perm])
    for name in ("w1", "w3", "w2"):
        a_ = getattr(inp, name)
        getattr(q, name)[...] = np.concatenate([a_[h * Eh:(h + 1) * Eh] for h in perm])
    out2 = O.forward(cfg, q)
    for i, h in enumerate(perm):
        assert np.allclose(out2["o"][:, i * dh:(i + 1) * dh], out["o"][:, h * dh:(h + 1) * dh],
                           rtol=1e-12, atol=1e-12)
    assert np.allclose(out2["y"], out["y"], rtol=1e-10, atol=1e-10)


def check_capacity_zero_and_xperm():
    """C = 0: every assignment dropped, y = u + s.  x_perm rows are the source rows."""
    O = _o()
    from moe_inputs import SMALL
    cfg = SMALL[2].with_(T=30, capacity=0)
    inp = _f32_inputs(cfg)
    out = O.forward(cfg, inp, want_xperm=True)
    x = O.decode(inp.x)
    assert out["offsets"][-1] == 0
    assert np.allclose(out["y"], x + out["s"], rtol=0, atol=0)
    cfg = SMALL[4].with_(T=25)
    inp = _f32_inputs(cfg)
    out = O.forward(cfg, inp, want_xperm=True)
    K = cfg.k_total
    for r, a in enumerate(out["src_of"]):
        t, j = divmod(int(a), K)
        h = int(out["topk_idx"][t, j]) // cfg.e_per_head
        assert np.array_equal(out["x_perm"][r], out["z"][t, h * cfg.d_head:(h + 1) * cfg.d_head])
    assert int(out["counts"].sum()) == cfg.T * K


ALL = [check_router_logits, check_softmax, check_topk, check_topk_groups, check_hand_example, check_capacity,
       check_affinity, check_permutation, check_ffn_library, check_dense_special_case,
       check_identical_experts, check_dense_masked, check_shared_concat,
       check_multihead_reductions, check_capacity_zero_and_xperm]
