"""Pins for the oracle's per-head RMSNorm of Q and K ("CuTeDSL at Perplexity",
section "QK Norm": every (token, head) pair of Q and of K is one row of
length head_dim, normalised on its own; Q rows take the Q weight, K rows the
K weight).

Every pin below is a fact fixed by that definition and the mathematics,
checked without retyping the oracle's formula:
  * closed forms: constant heads and one-hot heads, whose outputs are known
    exactly (eps = 0);
  * independence: changing one head leaves every other output bit-identical;
  * scale invariance of each head (eps = 0);
  * torch's float64 ``rms_norm`` over the last axis, a library routine for
    the same special case.
Plausible mistakes are planted in CPU copies of the oracle (weights swapped,
a token normalised over all its heads, axes transposed, a wrong divisor, a
reversed weight, K normalised with Q's rows); each must fail at least one pin.
"""

import math

import numpy as np
import pytest
import torch

from oracle import rownorm as O


def _heads(rng, T, nh, D, scale=1.0):
    return rng.standard_normal((T, nh, D)) * scale


# ---------------------------------------------------------------------------
# pins, each taking an implementation with the oracle's signature
# ---------------------------------------------------------------------------

def pin_constant_heads(impl):
    """A head of D equal values c != 0 has rms |c|: with eps = 0 its output is
    (w + b) sign(c) exactly, whatever the other heads hold."""
    rng = np.random.default_rng(1)
    T, nq, nk, D = 3, 4, 2, 16
    cq = rng.choice([-1.0, 1.0], (T, nq, 1)) * np.exp2(rng.integers(-20, 20, (T, nq, 1)))
    ck = rng.choice([-1.0, 1.0], (T, nk, 1)) * np.exp2(rng.integers(-20, 20, (T, nk, 1)))
    q = np.broadcast_to(cq, (T, nq, D)).copy()
    k = np.broadcast_to(ck, (T, nk, D)).copy()
    qw = rng.integers(-8, 8, D) / 4.0
    kw = rng.integers(-8, 8, D) / 4.0 + 3.0
    for b in (0.0, 1.0):
        qy, ky = impl(q, k, qw, kw, 0.0, b)
        if not (np.array_equal(qy, np.sign(cq) * (qw + b)) and np.array_equal(ky, np.sign(ck) * (kw + b))):
            return False
    return True


def pin_one_hot_heads(impl):
    """A head a * e_j has mean square a^2 / D: with eps = 0 its output is
    (w_j + b) sqrt(D) sign(a) at j and 0 elsewhere."""
    rng = np.random.default_rng(2)
    T, nq, nk, D = 2, 3, 3, 64
    q = np.zeros((T, nq, D))
    k = np.zeros((T, nk, D))
    jq = rng.integers(0, D, (T, nq))
    jk = rng.integers(0, D, (T, nk))
    aq = rng.choice([-3.0, 0.5, 7.0], (T, nq))
    ak = rng.choice([-2.0, 0.25, 5.0], (T, nk))
    for t in range(T):
        for h in range(nq):
            q[t, h, jq[t, h]] = aq[t, h]
        for h in range(nk):
            k[t, h, jk[t, h]] = ak[t, h]
    qw, kw = rng.standard_normal(D), rng.standard_normal(D)
    qy, ky = impl(q, k, qw, kw, 0.0, 0.0)
    for y, j, a, w, nh in ((qy, jq, aq, qw, nq), (ky, jk, ak, kw, nk)):
        for t in range(T):
            for h in range(nh):
                want = np.zeros(D)
                want[j[t, h]] = w[j[t, h]] * math.sqrt(D) * np.sign(a[t, h])
                if not np.allclose(y[t, h], want, rtol=1e-15, atol=0.0):
                    return False
    return True


def pin_small_closed_form(impl):
    """Head [3, 4] (D = 2): mean square 12.5, outputs 3 sqrt(2) / 5 and
    4 sqrt(2) / 5 (unit weight, eps = 0); as a K head with weight 2, twice that."""
    q = np.array([[[3.0, 4.0]]])
    k = np.array([[[3.0, 4.0]]])
    qy, ky = impl(q, k, np.array([1.0, 1.0]), np.array([2.0, 2.0]), 0.0, 0.0)
    want = np.array([3.0, 4.0]) * math.sqrt(2.0) / 5.0
    return np.allclose(qy[0, 0], want, rtol=1e-15) and np.allclose(ky[0, 0], 2 * want, rtol=1e-15)


def pin_heads_independent(impl):
    """Changing one head (values and scale) changes no other output bit."""
    rng = np.random.default_rng(3)
    T, nq, nk, D = 4, 5, 2, 32
    q, k = _heads(rng, T, nq, D), _heads(rng, T, nk, D, 2.0)
    qw, kw = rng.standard_normal(D), rng.standard_normal(D)
    eps = 1e-6
    qy, ky = impl(q, k, qw, kw, eps, 1.0)
    for (t, h, which) in ((1, 3, "q"), (2, 1, "k"), (0, 0, "q")):
        q2, k2 = q.copy(), k.copy()
        (q2 if which == "q" else k2)[t, h] = rng.standard_normal(D) * 100.0
        qy2, ky2 = impl(q2, k2, qw, kw, eps, 1.0)
        mq = np.ones(qy.shape, dtype=bool)
        mk = np.ones(ky.shape, dtype=bool)
        (mq if which == "q" else mk)[t, h] = False
        if not (np.array_equal(qy[mq], qy2[mq]) and np.array_equal(ky[mk], ky2[mk])):
            return False
        changed = (qy2 if which == "q" else ky2)[t, h]
        if np.array_equal(changed, (qy if which == "q" else ky)[t, h]):
            return False
    return True


def pin_scale_invariance(impl):
    """With eps = 0 each head's output does not change when the head is
    scaled by a positive power of two (exactly) or by any positive factor
    (to rounding)."""
    rng = np.random.default_rng(4)
    T, nq, nk, D = 3, 4, 4, 128
    q, k = _heads(rng, T, nq, D), _heads(rng, T, nk, D)
    s = np.exp2(rng.integers(-30, 30, (T, nq, 1))).astype(np.float64)
    qw, kw = rng.standard_normal(D), rng.standard_normal(D)
    qy, ky = impl(q, k, qw, kw, 0.0, 0.0)
    qy2, ky2 = impl(q * s, k * 3.7, qw, kw, 0.0, 0.0)
    return np.array_equal(qy, qy2) and np.allclose(ky, ky2, rtol=1e-13, atol=0.0)


def pin_torch_rms_norm(impl):
    """torch.nn.functional.rms_norm in float64 over the last axis of [T, H, D]
    with weight (w + b) is the same operation (eps values exact in float32,
    the precision the kernels take eps in)."""
    rng = np.random.default_rng(5)
    for T, nq, nk, D in ((7, 8, 2, 128), (3, 4, 4, 64), (2, 2, 1, 256)):
        q, k = _heads(rng, T, nq, D), _heads(rng, T, nk, D, 0.01)
        qw, kw = rng.standard_normal(D), rng.standard_normal(D)
        for eps, b in ((2.0 ** -20, 0.0), (2.0 ** -10, 1.0)):
            qy, ky = impl(q, k, qw, kw, eps, b)
            tq = torch.nn.functional.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(qw + b), eps).numpy()
            tk = torch.nn.functional.rms_norm(torch.from_numpy(k), (D,), torch.from_numpy(kw + b), eps).numpy()
            if not (np.allclose(qy, tq, rtol=1e-12, atol=1e-300) and np.allclose(ky, tk, rtol=1e-12, atol=1e-300)):
                return False
    return True


PINS = [pin_constant_heads, pin_one_hot_heads, pin_small_closed_form, pin_heads_independent, pin_scale_invariance,
        pin_torch_rms_norm]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_qknorm_pin(pin):
    assert pin(O.qknorm)


def test_qknorm_without_k():
    rng = np.random.default_rng(6)
    q, k = _heads(rng, 3, 4, 64), _heads(rng, 3, 2, 64)
    qw, kw = rng.standard_normal(64), rng.standard_normal(64)
    qy, _ = O.qknorm(q, k, qw, kw, 1e-6, 0.0)
    qy2, ky2 = O.qknorm(q, None, qw, None, 1e-6, 0.0)
    assert ky2 is None and np.array_equal(qy, qy2)


# ---------------------------------------------------------------------------
# planted mistakes (CPU copies of the oracle): each must fail some pin
# ---------------------------------------------------------------------------

def _rows_norm(t, w, eps, b, divisor=None):
    T, nh, D = t.shape
    x = t.reshape(T * nh, D)
    ms = (x * x).sum(axis=1) / (divisor if divisor else D)
    return ((w + b)[None, :] * x / np.sqrt(ms + eps)[:, None]).reshape(T, nh, D)


def mutant_swapped_weights(q, k, qw, kw, eps, b):
    return _rows_norm(q, kw, eps, b), None if k is None else _rows_norm(k, qw, eps, b)


def mutant_token_rows(q, k, qw, kw, eps, b):
    """normalises a token's heads together (one row per token)"""
    def one(t, w):
        T, nh, D = t.shape
        x = t.reshape(T, nh * D)
        ms = (x * x).sum(axis=1) / (nh * D)
        return (x / np.sqrt(ms + eps)[:, None]).reshape(T, nh, D) * (w + b)
    return one(q, qw), None if k is None else one(k, kw)


def mutant_transposed_axes(q, k, qw, kw, eps, b):
    """walks the heads in (head, token) order but writes back in (token, head) order"""
    def one(t, w):
        T, nh, D = t.shape
        y = _rows_norm(np.ascontiguousarray(t.transpose(1, 0, 2)), w, eps, b)
        return y.reshape(T, nh, D)
    return one(q, qw), None if k is None else one(k, kw)


def mutant_divisor_minus_one(q, k, qw, kw, eps, b):
    D = q.shape[2]
    return _rows_norm(q, qw, eps, b, D - 1), None if k is None else _rows_norm(k, kw, eps, b, D - 1)


def mutant_reversed_weight(q, k, qw, kw, eps, b):
    return _rows_norm(q, qw[::-1], eps, b), None if k is None else _rows_norm(k, kw[::-1], eps, b)


def mutant_k_uses_q_rows(q, k, qw, kw, eps, b):
    """K normalised with the mean squares of Q's rows at the same (token, head)"""
    qy = _rows_norm(q, qw, eps, b)
    if k is None:
        return qy, None
    nk = k.shape[1]
    msq = (q[:, :nk] ** 2).mean(axis=2, keepdims=True)
    return qy, (kw + b) * k / np.sqrt(msq + eps)


def mutant_bias_dropped(q, k, qw, kw, eps, b):
    return _rows_norm(q, qw, eps, 0.0), None if k is None else _rows_norm(k, kw, eps, 0.0)


MUTANTS = [mutant_swapped_weights, mutant_token_rows, mutant_transposed_axes, mutant_divisor_minus_one,
           mutant_reversed_weight, mutant_k_uses_q_rows, mutant_bias_dropped]


def test_correct_copy_passes_every_pin():
    """The helper the mutants are built from, unmutated, passes: the pins
    fail the mutants for their mistakes, not for the helper."""
    def good(q, k, qw, kw, eps, b):
        return _rows_norm(q, qw, eps, b), None if k is None else _rows_norm(k, kw, eps, b)
    assert all(p(good) for p in PINS)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_fails_some_pin(mutant):
    assert not all(p(mutant) for p in PINS)
