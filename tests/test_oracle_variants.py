"""The routing-variant oracle functions against their pins, and planted mistakes (CPU)."""
import numpy as np
import pytest

import oracle.moe_oracle as O
from tests import oracle_variant_pins as P


@pytest.mark.parametrize("check", P.ALL, ids=lambda f: f.__name__)
def test_variant_pin(check):
    check()


_orig = {n: getattr(O, n) for n in ("biased_keys", "biased_gates", "sel_bias_update", "seq_balance",
                                     "keep_expert_choice", "select_topk_keys")}


def m_bias_on_logits(p, sel_bias):
    # the bias added to log-probabilities instead of the probabilities
    return (np.log(np.asarray(p, np.float64)).astype(np.float32) + np.asarray(sel_bias, np.float32))


def m_bias_gate_ignored(p, sel_bias, idx, renorm, bias_in_gate):
    return _orig["biased_gates"](p, sel_bias, idx, renorm, 0)


def m_update_sign(sel_bias, counts, gamma):
    return _orig["sel_bias_update"](sel_bias, counts, -gamma)


def m_update_mean_strict(sel_bias, counts, gamma):
    # an expert at the mean treated as underloaded
    c = np.asarray(counts, np.int64)
    step = np.where(c * len(c) > c.sum(), -1.0, 1.0).astype(np.float32)
    return (np.asarray(sel_bias, np.float32) + np.float32(gamma) * step).astype(np.float32)


def m_seq_over_k(p, idx, seq_len):
    return _orig["seq_balance"](p, idx, seq_len) / idx.shape[1]


def m_seq_whole_batch(p, idx, seq_len):
    v = _orig["seq_balance"](p, idx, p.shape[0])
    return np.full(p.shape[0] // int(seq_len), v[0])


def m_ec_ties_high(e_flat, w32_flat, n_experts, C):
    kept = np.zeros(len(e_flat), bool)
    for e in range(n_experts):
        m = np.nonzero(e_flat == e)[0].tolist()
        kept[sorted(m, key=lambda a: (-float(w32_flat[a]), -a))[:min(C, len(m))]] = True
    return kept


def m_ec_plus_one(e_flat, w32_flat, n_experts, C):
    return _orig["keep_expert_choice"](e_flat, w32_flat, n_experts, C + 1)


def m_keys_ties_high(keys, k, n_groups=0, topk_groups=0):
    keys = np.asarray(keys, np.float32)[:, ::-1]
    E = keys.shape[1]
    return (E - 1 - O.select_topk(keys, k, 0, 0)).astype(np.int32) if not n_groups else \
        _orig["select_topk_keys"](keys[:, ::-1], k, n_groups, topk_groups)


MUTANTS = [("biased_keys", m_bias_on_logits), ("biased_gates", m_bias_gate_ignored),
           ("sel_bias_update", m_update_sign), ("sel_bias_update", m_update_mean_strict),
           ("seq_balance", m_seq_over_k), ("seq_balance", m_seq_whole_batch),
           ("keep_expert_choice", m_ec_ties_high), ("keep_expert_choice", m_ec_plus_one),
           ("select_topk_keys", m_keys_ties_high)]


@pytest.mark.parametrize("name,mut", MUTANTS, ids=lambda v: getattr(v, "__name__", str(v)))
def test_variant_mutant_caught(name, mut, monkeypatch):
    monkeypatch.setattr(O, name, mut)
    caught = []
    for check in P.ALL:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin caught {mut.__name__} in {name}"
