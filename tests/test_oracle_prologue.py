"""The oracle's fused input prologue (packed qkv split, L2 normalisation, gate
activations) against closed forms, invariants and position codes, plus planted
mistakes (monkeypatched into the oracle module, on the CPU) that each must make at
least one of these pins fail."""
import math

import numpy as np
import pytest

import oracle

LN3 = math.log(3.0)


def pin_gate_closed_forms():
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4; exp(-softplus(ln 3)) = 1 / (1 + 3) = 1/4
    x = np.array([LN3, -LN3, 0.0])
    np.testing.assert_allclose(oracle.sigmoid(x), [0.75, 0.25, 0.5], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.decay_from_logit(x), [0.25, 0.75, 0.5], rtol=0, atol=1e-15)


def pin_gate_complement():
    # exp(-softplus(x)) = 1 / (1 + e^x) = 1 - sigmoid(x); sigmoid rises, the decay falls
    x = np.linspace(-30.0, 30.0, 601)
    b, a = oracle.sigmoid(x), oracle.decay_from_logit(x)
    np.testing.assert_allclose(a + b, 1.0, rtol=0, atol=2e-15)
    assert np.all(np.diff(b) > 0) and np.all(np.diff(a) < 0)
    assert np.all((b > 0) & (b < 1) & (a > 0) & (a < 1))


def pin_gate_extremes():
    with np.errstate(over="raise", invalid="raise"):
        b = oracle.sigmoid(np.array([1000.0, -1000.0]))
        a = oracle.decay_from_logit(np.array([1000.0, -1000.0]))
    assert b[0] == 1.0 and b[1] == 0.0
    assert a[0] == 0.0 and a[1] == 1.0


def pin_l2_examples():
    np.testing.assert_allclose(oracle.l2_normalize(np.array([3.0, 4.0])), [0.6, 0.8], rtol=0, atol=1e-16)
    assert np.all(oracle.l2_normalize(np.zeros((2, 5))) == 0.0)  # a zero row stays zero
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.01, 100.0, (7, 3, 1))
    y = oracle.l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.l2_normalize(37.5 * x), y, rtol=1e-14, atol=1e-16)
    # the direction is kept: y is a positive multiple of x
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-14)


def pin_unpack_layout():
    # element j of token t of batch b encodes (b, t, j); the split must put q of
    # head h at j = h dk + i, k at H dk + h dk + i, v at 2 H dk + h dv + i
    B, T, H, dk, dv, pad = 2, 3, 2, 4, 3, 5
    W = 2 * H * dk + H * dv + pad
    bb, tt, jj = np.meshgrid(np.arange(B), np.arange(T), np.arange(W), indexing="ij")
    qkv = 1e6 * bb + 1e3 * tt + jj
    q, k, v = oracle.unpack_qkv(qkv, H, dk, dv)
    assert q.shape == (B, T, H, dk) and k.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for i in range(dk):
                    assert q[b, t, h, i] == 1e6 * b + 1e3 * t + h * dk + i
                    assert k[b, t, h, i] == 1e6 * b + 1e3 * t + H * dk + h * dk + i
                for i in range(dv):
                    assert v[b, t, h, i] == 1e6 * b + 1e3 * t + 2 * H * dk + h * dv + i


def _packed(q, k, v):
    B, T, H, dk = q.shape
    return np.concatenate([q.reshape(B, T, H * dk), k.reshape(B, T, H * dk), v.reshape(B, T, -1)], axis=-1)


def pin_prologue_single_token():
    # one token from zero state: S = b v k^^T, o = b (k^ . q^) v / sqrt(dk); with q and
    # k along the same unit vector u (scaled by 5 and 0.5) k^ . q^ = 1, and
    # x_b = ln 3 gives b = 3/4 exactly
    dk, dv = 8, 5
    rng = np.random.default_rng(1)
    u = rng.standard_normal(dk)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(dv)
    q = (5.0 * u).reshape(1, 1, 1, dk)
    k = (0.5 * u).reshape(1, 1, 1, dk)
    qkv = _packed(q, k, v.reshape(1, 1, 1, dv))
    out, st = oracle.forward_packed(qkv, np.full((1, 1, 1), LN3), np.full((1, 1, 1), -7.0), 1, dk, dv)
    np.testing.assert_allclose(out[0, 0, 0], 0.75 * v / math.sqrt(dk), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], 0.75 * np.outer(v, u), rtol=1e-13, atol=1e-15)


def pin_prologue_decay_through_recurrence():
    # two tokens with orthogonal keys e0, e1 (scaled by 3 and 0.25): k^_2 . S_1 = 0,
    # so S_2 = a_2 S_1 + b_2 v_2 e1^T; a query along e0 reads a_2 b_1 v_1.  x_b1 = 0
    # gives b_1 = 1/2, x_a2 = ln 3 gives a_2 = 1/4: o_2 = v_1 / (8 sqrt(dk)).
    dk, dv = 4, 3
    e0, e1 = np.eye(dk)[0], np.eye(dk)[1]
    v1, v2 = np.array([1.0, -2.0, 0.5]), np.array([4.0, 0.25, -1.0])
    q = np.stack([e1, 7.0 * e0]).reshape(1, 2, 1, dk)
    k = np.stack([3.0 * e0, 0.25 * e1]).reshape(1, 2, 1, dk)
    v = np.stack([v1, v2]).reshape(1, 2, 1, dv)
    xb = np.array([0.0, 1.3]).reshape(1, 2, 1)
    xa = np.array([-2.0, LN3]).reshape(1, 2, 1)
    out, _ = oracle.forward_packed(_packed(q, k, v), xb, xa, 1, dk, dv)
    np.testing.assert_allclose(out[0, 1, 0], v1 / (8.0 * math.sqrt(dk)), rtol=1e-13, atol=1e-15)


PINS = [pin_gate_closed_forms, pin_gate_complement, pin_gate_extremes, pin_l2_examples, pin_unpack_layout,
        pin_prologue_single_token, pin_prologue_decay_through_recurrence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prologue_pin(pin):
    pin()


def _decay_sign(x):
    x = np.asarray(x, np.float64)
    return np.exp(-np.logaddexp(0.0, -x))


def _sigmoid_sign(x):
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(x))


def _l1(x, eps=1e-12):
    x = np.asarray(x, np.float64)
    return x / np.maximum(np.sum(np.abs(x), axis=-1, keepdims=True), eps)


def _unpack_swapped(qkv, H, dk, dv):
    q, k, v = _ORIG["unpack_qkv"](qkv, H, dk, dv)
    return k, q, v


def _unpack_head_major(qkv, H, dk, dv):
    # reads each head's q, k, v side by side ([h][q k v] instead of [q][k][v])
    x = np.asarray(qkv, np.float64)
    B, T, _ = x.shape
    per = x[:, :, :H * (2 * dk + dv)].reshape(B, T, H, 2 * dk + dv)
    return (np.ascontiguousarray(per[..., :dk]), np.ascontiguousarray(per[..., dk:2 * dk]),
            np.ascontiguousarray(per[..., 2 * dk:]))


def _prologue_no_q_norm(qkv, beta_logit, decay_logit, H, dk, dv):
    q, k, v = oracle.unpack_qkv(qkv, H, dk, dv)
    return dict(q=q, k=oracle.l2_normalize(k), v=v, beta=oracle.sigmoid(beta_logit),
                decay=oracle.decay_from_logit(decay_logit))


def _prologue_raw_gates(qkv, beta_logit, decay_logit, H, dk, dv):
    q, k, v = oracle.unpack_qkv(qkv, H, dk, dv)
    return dict(q=oracle.l2_normalize(q), k=oracle.l2_normalize(k), v=v, beta=np.asarray(beta_logit, np.float64),
                decay=np.asarray(decay_logit, np.float64))


_ORIG = {name: getattr(oracle, name) for name in ("unpack_qkv", "l2_normalize", "sigmoid", "decay_from_logit",
                                                  "prologue")}

MUTANTS = [
    ("decay_sign", "decay_from_logit", _decay_sign),
    ("sigmoid_sign", "sigmoid", _sigmoid_sign),
    ("l1_norm", "l2_normalize", _l1),
    ("q_k_swapped", "unpack_qkv", _unpack_swapped),
    ("head_major_split", "unpack_qkv", _unpack_head_major),
    ("q_not_normalised", "prologue", _prologue_no_q_norm),
    ("logits_as_values", "prologue", _prologue_raw_gates),
]


@pytest.mark.parametrize("name,attr,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_prologue_pins_catch_planted_mistake(name, attr, fn, monkeypatch):
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no prologue pin caught the planted mistake {name}"
