"""The backward oracle against finite differences and special cases, and planted mistakes (CPU)."""
import numpy as np
import pytest

import oracle.moe_backward as B
from tests import oracle_backward_pins as P


@pytest.mark.parametrize("check", P.ALL, ids=lambda f: f.__name__)
def test_backward_pin(check):
    check()


def _all_pass():
    for c in P.ALL:
        c()


# ---------------------------------------------------------------- mutants
def m_silu_grad_is_sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


_orig_backward = B.backward


def m_no_renorm_correction(cfg, P_, topk_idx, kept, dy, lam=0.0, seq_w=0.0):
    return _orig_backward(cfg.with_(renorm=0), P_, topk_idx, kept, dy, lam, seq_w) if cfg.renorm else \
        _orig_backward(cfg, P_, topk_idx, kept, dy, lam, seq_w)


def m_aux_over_S(cfg, P_, topk_idx, kept, dy, lam=0.0, seq_w=0.0):
    # aux gradient scaled by 1/S instead of 1/S^2
    return _orig_backward(cfg, P_, topk_idx, kept, dy, lam * cfg.T, seq_w)


def m_seq_over_L(cfg, P_, topk_idx, kept, dy, lam=0.0, seq_w=0.0):
    # sequence-term gradient scaled by 1/L instead of 1/L^2
    return _orig_backward(cfg, P_, topk_idx, kept, dy, lam, seq_w * (cfg.seq_len or 1))


def m_mlp_transposed(act, v, w1, w3, w2, dF):
    dv, dW1, dW3, dW2 = _orig_mlp(act, v, w1, w3, w2, dF)
    return dv, dW1, dW3, dW2 * 0.5 + dW2[..., ::-1] * 0.5 if dW2.shape[-1] > 1 else dW2 * 0.9


_orig_mlp = B._mlp_backward


def m_global_softmax_jacobian(cfg, p, dp):
    # the Jacobian taken over all experts instead of each head's own
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


@pytest.mark.parametrize("name,target,repl", [
    ("silu_grad", "_silu_grad", m_silu_grad_is_sigmoid),
    ("renorm", "backward", m_no_renorm_correction),
    ("aux_scale", "backward", m_aux_over_S),
    ("seq_scale", "backward", m_seq_over_L),
    ("dw2_mixed", "_mlp_backward", m_mlp_transposed),
    ("global_softmax", "_head_softmax_backward", m_global_softmax_jacobian),
])
def test_backward_mutant_caught(monkeypatch, name, target, repl):
    monkeypatch.setattr(B, target, repl)
    with pytest.raises(AssertionError):
        _all_pass()
