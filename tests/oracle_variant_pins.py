"""Checks that pin the routing-variant functions of the oracle to facts outside it.

What pins what (CPU only):
  biased selection   the hand-worked example in golden/hand_variants.json; a
                     brute-force subset search on float32 keys p + b with
                     forced ties; a zero bias reduces to the plain router; a
                     bias larger than any probability forces its expert first;
                     the group-limited form by brute force over group subsets
  biased gates       the hand example (bias in the gate or not)
  bias update        the hand example; balanced loads leave the bias alone;
                     every step is exactly -gamma, 0 or +gamma
  sequence balance   the hand example (two sequences); one sequence equals the
                     GShard aux value of the same batch (the 4-token example:
                     0.5375); invariant under reordering tokens inside a
                     sequence
  expert choice      the hand example; a brute-force rank count with forced
                     ties; every expert keeps exactly min(C, T); C >= T gives
                     the dense softmax mixture sum_e p_e FFN_e(u) (the
                     "Adaptive Mixtures of Local Experts" output), checked
                     against torch
Each check raises AssertionError on failure; test_oracle_variants.py runs them
and plants mistakes that they must catch.
"""
import itertools
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _o():
    import oracle.moe_oracle as O
    return O


def golden():
    with open(os.path.join(HERE, "golden", "hand_variants.json")) as f:
        return json.load(f)


def _before(key, a, b):
    """Does (key[a], -a) beat (key[b], -b)?"""
    return key[a] > key[b] or (key[a] == key[b] and a < b)


def _brute_topk_keys(key, k, allowed=None):
    E = len(key)
    cand = [e for e in range(E) if allowed is None or allowed[e]]
    for sub in itertools.combinations(cand, k):
        rest = [e for e in cand if e not in sub]
        if all(_before(key, a, b) for a in sub for b in rest):
            return sorted(sub, key=lambda e: (-float(key[e]), e))
    raise AssertionError("no subset satisfies the order")


def check_biased_hand():
    O = _o()
    g = golden()["biased"]
    p = np.array(g["probs"], np.float64)
    b = np.array(g["sel_bias"], np.float32)
    keys = O.biased_keys(p, b)
    idx = O.select_topk_keys(keys, g["k"])
    assert idx.tolist() == g["topk_idx"], idx
    plain = O.select_topk(np.log(p).astype(np.float32), g["k"])
    assert plain.tolist() == g["plain_topk_idx"]
    w0 = O.biased_gates(p, b, idx, 0, 0)
    w1 = O.biased_gates(p, b, idx, 0, 1)
    assert np.array_equal(w0, np.array(g["gates_bias_not_in_gate"])), w0
    assert np.array_equal(w1, np.array(g["gates_bias_in_gate"])), w1


def check_biased_bruteforce():
    O = _o()
    rng = np.random.default_rng(5)
    for trial in range(40):
        E, k = 7, 1 + trial % 4
        p = rng.dirichlet(np.ones(E), size=6)
        b = (rng.integers(-3, 4, size=E) * 0.01).astype(np.float32)
        if trial % 3 == 0:  # force exact ties of the float32 keys
            p[:, 2] = p[:, 5]
            b[2] = b[5]
        keys = O.biased_keys(p, b)
        idx = O.select_topk_keys(keys, k)
        for t in range(len(p)):
            # the key is the float32 sum of the float32 probability and the bias
            key = [np.float32(np.float32(p[t, e]) + b[e]) for e in range(E)]
            assert list(idx[t]) == _brute_topk_keys(key, k), (trial, t)


def check_biased_groups():
    O = _o()
    rng = np.random.default_rng(6)
    G, gsz, gk, k = 4, 3, 2, 3
    E = G * gsz
    for trial in range(30):
        p = rng.dirichlet(np.ones(E), size=5)
        b = (rng.integers(-4, 5, size=E) * 0.01).astype(np.float32)
        keys = O.biased_keys(p, b)
        idx = O.select_topk_keys(keys, k, G, gk)
        for t in range(len(p)):
            key = [float(v) for v in keys[t]]
            gs = [max(key[g * gsz:(g + 1) * gsz]) for g in range(G)]
            gsel = _brute_topk_keys(gs, gk)
            allowed = [e // gsz in gsel for e in range(E)]
            assert list(idx[t]) == _brute_topk_keys(key, k, allowed), (trial, t)


def check_biased_reductions():
    O = _o()
    rng = np.random.default_rng(7)
    E, k = 9, 3
    l = rng.standard_normal((50, E)).astype(np.float32)
    p = O.softmax(l)
    zero = np.zeros(E, np.float32)
    # no bias: the plain router (selection on the logits)
    assert np.array_equal(O.select_topk_keys(O.biased_keys(p, zero), k), O.select_topk(l, k))
    idx = O.select_topk(l, k)
    assert np.array_equal(O.biased_gates(p, zero, idx, 0, 1), O.gates(p, idx, 0))
    assert np.array_equal(O.biased_gates(p, zero, idx, 1, 1), O.gates(p, idx, 1))
    # a bias above every probability puts its expert first for every token
    big = zero.copy()
    big[4] = 2.0
    idx = O.select_topk_keys(O.biased_keys(p, big), k)
    assert np.all(idx[:, 0] == 4)
    assert np.allclose(O.biased_gates(p, big, idx, 0, 1)[:, 0], p[:, 4] + 2.0, rtol=0, atol=1e-15)
    assert np.array_equal(O.biased_gates(p, big, idx, 0, 0)[:, 0], p[:, 4])


def check_bias_update():
    O = _o()
    g = golden()["bias_update"]
    got = O.sel_bias_update(np.array(g["sel_bias"], np.float32), np.array(g["counts"]), g["gamma"])
    assert np.array_equal(got, np.array(g["updated"], np.float32)), got
    b = np.array([0.01, -0.02, 0.0], np.float32)
    assert np.array_equal(O.sel_bias_update(b, np.array([4, 4, 4]), 0.001), b)
    rng = np.random.default_rng(8)
    for _ in range(20):
        c = rng.integers(0, 9, size=6)
        b = (rng.integers(-5, 6, size=6) * 0.001).astype(np.float32)
        step = O.sel_bias_update(b, c, 0.001) - b
        mean = c.sum() / 6.0
        for e in range(6):
            want = 0.0 if c[e] == mean else (0.001 if c[e] < mean else -0.001)
            assert abs(step[e] - want) < 1e-9, (c, e, step)


def check_seq_balance():
    O = _o()
    g = golden()["seq_balance"]
    v = O.seq_balance(np.array(g["probs"]), np.array(g["topk_idx"]), g["seq_len"])
    assert np.allclose(v, g["values"], rtol=0, atol=1e-15), v
    # one sequence: the GShard aux value of the same batch (hand example 0.5375)
    from tests.oracle_pins import golden as g4
    h = g4()
    p4, i4 = np.array(h["probs"]), np.array(h["topk_idx"])
    assert abs(O.seq_balance(p4, i4, 4)[0] - h["aux"]) < 1e-15
    rng = np.random.default_rng(9)
    p = rng.dirichlet(np.ones(6), size=24)
    idx = O.select_topk(np.log(p).astype(np.float32), 2)
    assert abs(O.seq_balance(p, idx, 24)[0] - O.aux_loss(p, idx)) < 1e-14
    # reordering the tokens inside each sequence changes nothing
    perm = np.concatenate([rng.permutation(8) + 8 * s for s in range(3)])
    assert np.allclose(O.seq_balance(p, idx, 8), O.seq_balance(p[perm], idx[perm], 8), rtol=1e-14, atol=0)


def check_expert_choice_hand():
    O = _o()
    from moe_inputs import MoEConfig
    g = golden()["expert_choice"]
    p = np.array(g["probs"])
    T, E = p.shape
    cfg = MoEConfig("ec_hand", T=T, d_model=64, n_heads=1, d_head=64, n_experts=E, top_k=1,
                    drop=1, capacity=g["capacity"], d_ff=64, route_mode=1)
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    kp = O.keep(cfg, idx, p.astype(np.float32))
    assert kp["counts"].tolist() == g["counts"]
    assert kp["offsets"].tolist() == g["offsets"]
    assert kp["src_of"].tolist() == g["src_of"]
    assert kp["row_of"].tolist() == g["row_of"]


def check_expert_choice_bruteforce():
    O = _o()
    rng = np.random.default_rng(10)
    for trial in range(30):
        T, E, C = 11, 4, 1 + trial % 6
        w = rng.dirichlet(np.ones(E), size=T).astype(np.float32)
        if trial % 2 == 0:  # ties inside expert columns
            w[3] = w[7]
            w[9, 1] = w[0, 1]
        e_flat = np.tile(np.arange(E), T)
        kept = O.keep_expert_choice(e_flat, w.reshape(-1), E, C)
        for t in range(T):
            for e in range(E):
                better = sum(1 for u in range(T) if w[u, e] > w[t, e] or (w[u, e] == w[t, e] and u < t))
                assert kept[t * E + e] == (better < C), (trial, t, e)
        assert np.all(kept.reshape(T, E).sum(axis=0) == min(C, T))


def check_expert_choice_dense():
    """C >= T: every expert takes every token; y = u + sum_e p_e FFN_e(u) (torch)."""
    O = _o()
    from moe_inputs import MoEConfig, generate
    from tests.oracle_pins import _torch_ffn
    for act in (0, 1):
        cfg = MoEConfig("ec_dense", T=9, d_model=64, n_heads=1, d_head=64, n_experts=3, top_k=1,
                        drop=1, capacity=9, d_ff=64, act=act, act_dtype=0, router_dtype=0, route_mode=1, tag=31)
        inp = generate(cfg)
        out = O.forward(cfg, inp)
        assert np.all(out["counts"] == cfg.T)
        x = O.decode(inp.x)
        l = x @ O.decode(inp.w_router).T
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        ref = x.copy()
        for e in range(cfg.n_experts):
            f = _torch_ffn(x, O.decode(inp.w1[e]), O.decode(inp.w3[e]) if act else None, O.decode(inp.w2[e]), act)
            ref += p[:, e:e + 1] * f
        assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-6)


ALL = [check_biased_hand, check_biased_bruteforce, check_biased_groups, check_biased_reductions,
       check_bias_update, check_seq_balance, check_expert_choice_hand, check_expert_choice_bruteforce,
       check_expert_choice_dense]
