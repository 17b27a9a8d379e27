"""Pins for the CPU oracle: checks against what the mathematics fixes, independent of
the oracle's own loops (closed forms, invariants, special cases that reduce to a
textbook rule, brute force on tiny inputs, and a hand-worked example).

Every pin takes the loaded oracle library as ``lib`` so that the same battery can be
run against deliberately broken copies of the oracle (see test_oracle.py): each
planted mistake must make at least one pin fail.

The recurrence (gated delta rule), per (batch, head):
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t / sqrt(d_k).
"""
from __future__ import annotations

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(B=1, T=24, H=2, dk=8, dv=6, seed=0, a_lo=0.3, a_hi=1.0, unit_k=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    decay = rng.uniform(a_lo, a_hi, (B, T, H))
    s0 = rng.standard_normal((B, H, dv, dk))
    return q, k, v, beta, decay, s0


def _close(x, y, tol=1e-12, what=""):
    r = oracle.rel_l2(x, y)
    assert r <= tol, f"{what}: rel-L2 {r:.3e} > {tol:.0e}"


# -- (i) b = 0 and S0 = 0: nothing is ever written -----------------------------------
def pin_zero_write_zero_state(lib):
    q, k, v, beta, decay, _ = rand_case(seed=1)
    beta[:] = 0.0
    for fn in (oracle.forward, oracle.dense):
        out, st = fn(q, k, v, beta, decay, None, lib=lib)
        assert np.all(out == 0.0) and np.all(st == 0.0), fn.__name__
    out, st = oracle.chunkwise(q, k, v, beta, decay, None, chunk=5, lib=lib)
    assert np.all(out == 0.0) and np.all(st == 0.0), "chunkwise"
    assert np.all(oracle.bidi(q, k, v, beta, decay, lib=lib) == 0.0), "bidi"


# -- (ii) b = 0, S0 != 0: the state only decays: S_t = (a_1...a_t) S0 ------------------
def pin_zero_write_decays_state(lib):
    q, k, v, beta, decay, s0 = rand_case(B=2, T=20, H=3, dk=8, dv=5, seed=2)
    beta[:] = 0.0
    cp = np.cumprod(decay, axis=1)  # [B,T,H]
    # o_t = cp_t * S0 q_t / sqrt(dk)
    exp_out = np.einsum("bth,bhij,bthj->bthi", cp, s0, q) / np.sqrt(8)
    exp_st = cp[:, -1, :, None, None] * s0
    for fn in (oracle.forward, oracle.dense):
        out, st = fn(q, k, v, beta, decay, s0, lib=lib)
        _close(out, exp_out, what=fn.__name__ + " out")
        _close(st, exp_st, what=fn.__name__ + " state")
    out, st = oracle.chunkwise(q, k, v, beta, decay, s0, chunk=7, lib=lib)
    _close(out, exp_out, what="chunkwise out")
    _close(st, exp_st, what="chunkwise state")


# -- (iii) T = 1, S0 = 0: o = b v (k.q) / sqrt(dk), state = b v k^T -------------------
def pin_single_token(lib):
    q, k, v, beta, decay, _ = rand_case(B=1, T=1, H=3, dk=16, dv=4, seed=3)
    exp_out = beta[..., None] * v * np.sum(k * q, axis=-1, keepdims=True) / 4.0
    exp_st = np.einsum("bh,bhi,bhj->bhij", beta[:, 0], v[:, 0], k[:, 0])
    for fn in (oracle.forward, oracle.dense):
        out, st = fn(q, k, v, beta, decay, None, lib=lib)
        _close(out, exp_out, what=fn.__name__)
        _close(st, exp_st, what=fn.__name__ + " state")
    out, st = oracle.chunkwise(q, k, v, beta, decay, None, chunk=4, lib=lib)
    _close(out, exp_out, what="chunkwise")


def _orthonormal(d, seed):
    rng = np.random.default_rng(seed)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Qm.T  # rows are orthonormal keys


def _key_schedule(T, d, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, d, T), rng.integers(0, d, T)  # write key, query key


# -- (iv) a = 1, b = 1, orthonormal keys: querying k_i returns the latest value -------
def pin_associative_recall(lib):
    dk, dv, T = 16, 5, 48
    keys = _orthonormal(dk, 4)
    wi, qi = _key_schedule(T, dk, 5)
    rng = np.random.default_rng(6)
    v = rng.standard_normal((1, T, 1, dv))
    k = keys[wi][None, :, None, :]
    q = keys[qi][None, :, None, :]
    beta = np.ones((1, T, 1))
    decay = np.ones((1, T, 1))
    memory = {}
    expect = np.zeros((T, dv))
    for t in range(T):
        memory[int(wi[t])] = v[0, t, 0]
        expect[t] = memory.get(int(qi[t]), np.zeros(dv))
    for fn in (oracle.forward, oracle.dense):
        out, _ = fn(q, k, v, beta, decay, None, lib=lib)
        got = out[0, :, 0] * np.sqrt(dk)
        assert np.max(np.abs(got - expect)) < 1e-12, fn.__name__


# -- (v) b = 1, general a, orthonormal keys: the write is then decayed by later a's ---
def pin_decayed_recall(lib):
    dk, dv, T = 8, 3, 40
    keys = _orthonormal(dk, 7)
    wi, qi = _key_schedule(T, dk, 8)
    rng = np.random.default_rng(9)
    v = rng.standard_normal((1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dv, dk))
    a = rng.uniform(0.5, 1.0, T)
    k = keys[wi][None, :, None, :]
    q = keys[qi][None, :, None, :]
    beta = np.ones((1, T, 1))
    decay = a[None, :, None].copy()
    # value read back from key i: initial S0 k_i decayed by every a, or the last
    # write v_s decayed by a_{s+1} ... a_t (the write itself is not decayed by a_s)
    memory = {i: s0[0, 0] @ keys[i] for i in range(dk)}
    expect = np.zeros((T, dv))
    for t in range(T):
        for i in memory:
            memory[i] = memory[i] * a[t]
        memory[int(wi[t])] = v[0, t, 0].copy()
        expect[t] = memory[int(qi[t])]
    for fn in (oracle.forward, oracle.dense):
        out, _ = fn(q, k, v, beta, decay, s0, lib=lib)
        got = out[0, :, 0] * np.sqrt(dk)
        assert np.max(np.abs(got - expect)) < 1e-12, fn.__name__


# -- (vi) a single repeated key: S k follows a scalar EMA; S q_perp only decays ------
def pin_single_key_ema(lib):
    dk, dv, T = 6, 4, 30
    rng = np.random.default_rng(10)
    kv = rng.standard_normal(dk)
    kv /= np.linalg.norm(kv)
    qp = rng.standard_normal(dk)
    qp -= (qp @ kv) * kv
    qp /= np.linalg.norm(qp)
    k = np.broadcast_to(kv, (1, T, 1, dk)).copy()
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0, 1, (1, T, 1))
    decay = rng.uniform(0.2, 1, (1, T, 1))
    s0 = rng.standard_normal((1, 1, dv, dk))
    m = s0[0, 0] @ kv
    for t in range(T):
        m = decay[0, t, 0] * (1.0 - beta[0, t, 0]) * m + beta[0, t, 0] * v[0, t, 0]
    perp = np.prod(decay[0, :, 0]) * (s0[0, 0] @ qp)
    for fn in (oracle.forward, oracle.dense):
        _, st = fn(q, k, v, beta, decay, s0, lib=lib)
        assert np.max(np.abs(st[0, 0] @ kv - m)) < 1e-12, fn.__name__
        assert np.max(np.abs(st[0, 0] @ qp - perp)) < 1e-12, fn.__name__


# -- (vii) a = 1: the Widrow-Hoff / LMS delta rule, which learns a consistent linear map
def pin_lms_learns_linear_map(lib):
    dk, dv = 6, 3
    rng = np.random.default_rng(11)
    Mtrue = rng.standard_normal((dv, dk))
    keys = rng.standard_normal((dk, dk))
    keys /= np.linalg.norm(keys, axis=1, keepdims=True)
    epochs = 400
    T = epochs * dk
    k = np.tile(keys, (epochs, 1))[None, :, None, :]
    v = (k[0, :, 0] @ Mtrue.T)[None, :, None, :]
    q = k.copy()
    beta = np.full((1, T, 1), 0.9)
    decay = np.ones((1, T, 1))
    _, st = oracle.forward(q, k, v, beta, decay, None, lib=lib)
    assert oracle.rel_l2(st[0, 0], Mtrue) < 1e-8, oracle.rel_l2(st[0, 0], Mtrue)


# -- (viii) linearity in (v, S0) at fixed q, k, a, b -----------------------------------
def pin_linearity(lib):
    q, k, v1, beta, decay, s1 = rand_case(B=1, T=30, H=2, dk=8, dv=5, seed=12)
    _, _, v2, _, _, s2 = rand_case(B=1, T=30, H=2, dk=8, dv=5, seed=13)
    o1, t1 = oracle.forward(q, k, v1, beta, decay, s1, lib=lib)
    o2, t2 = oracle.forward(q, k, v2, beta, decay, s2, lib=lib)
    o3, t3 = oracle.forward(q, k, v1 + 2.5 * v2, beta, decay, s1 + 2.5 * s2, lib=lib)
    _close(o3, o1 + 2.5 * o2, 1e-12, "linearity out")
    _close(t3, t1 + 2.5 * t2, 1e-12, "linearity state")


# -- (ix) rows of S are independent: permuting d_v permutes the output exactly --------
def pin_row_independence(lib):
    q, k, v, beta, decay, s0 = rand_case(B=1, T=25, H=2, dk=8, dv=7, seed=14)
    perm = np.random.default_rng(15).permutation(7)
    o, st = oracle.forward(q, k, v, beta, decay, s0, lib=lib)
    op, stp = oracle.forward(q, k, v[..., perm], beta, decay, s0[:, :, perm, :], lib=lib)
    assert np.array_equal(op, o[..., perm]) and np.array_equal(stp, st[:, :, perm, :])


# -- (x) streaming: splitting the sequence and carrying the state is exact ------------
def pin_streaming_split(lib):
    q, k, v, beta, decay, s0 = rand_case(B=2, T=40, H=2, dk=8, dv=6, seed=16)
    o, st = oracle.forward(q, k, v, beta, decay, s0, lib=lib)
    cuts = [0, 7, 8, 23, 40]
    s = s0
    parts = []
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        sl = slice(a_, b_)
        oo, s = oracle.forward(q[:, sl], k[:, sl], v[:, sl], beta[:, sl], decay[:, sl], s, lib=lib)
        parts.append(oo)
    assert np.array_equal(np.concatenate(parts, axis=1), o) and np.array_equal(s, st)
    # an empty call carries the state through unchanged
    oo, s_empty = oracle.forward(q[:, :0], k[:, :0], v[:, :0], beta[:, :0], decay[:, :0], s0, lib=lib)
    assert oo.shape[1] == 0 and np.array_equal(s_empty, s0)


# -- (xi) bidirectional: fwd + reversed fwd; symmetric under time reversal ------------
def pin_bidi(lib):
    q, k, v, beta, decay, _ = rand_case(B=1, T=33, H=2, dk=8, dv=5, seed=17)
    ob = oracle.bidi(q, k, v, beta, decay, lib=lib)
    f, _ = oracle.forward(q, k, v, beta, decay, None, lib=lib)
    R = lambda x: np.ascontiguousarray(x[:, ::-1])
    r, _ = oracle.forward(R(q), R(k), R(v), R(beta), R(decay), None, lib=lib)
    assert np.array_equal(ob, f + R(r)), "bidi != fwd + R fwd R"
    ob_rev = oracle.bidi(R(q), R(k), R(v), R(beta), R(decay), lib=lib)
    assert np.array_equal(ob_rev, R(ob)), "bidi(R x) != R bidi(x)"
    # a single token is seen by both directions: twice the causal output
    ob1 = oracle.bidi(q[:, :1], k[:, :1], v[:, :1], beta[:, :1], decay[:, :1], lib=lib)
    _close(ob1, 2.0 * f[:, :1], 1e-15, "bidi T=1")


# -- (xii) chunked and dense forms agree with the sequential form ---------------------
def pin_forms_agree(lib):
    cases = [
        dict(B=1, T=37, H=2, dk=8, dv=6, seed=18),
        dict(B=2, T=64, H=1, dk=16, dv=16, seed=19),
    ]
    for c in cases:
        q, k, v, beta, decay, s0 = rand_case(**c)
        o, st = oracle.forward(q, k, v, beta, decay, s0, lib=lib)
        for C in (1, 3, 16, 64):
            oc, sc = oracle.chunkwise(q, k, v, beta, decay, s0, chunk=C, lib=lib)
            _close(oc, o, 1e-12, f"chunkwise C={C}")
            _close(sc, st, 1e-12, f"chunkwise C={C} state")
        od, sd = oracle.dense(q[:, :20], k[:, :20], v[:, :20], beta[:, :20], decay[:, :20], s0, lib=lib)
        o20, s20 = oracle.forward(q[:, :20], k[:, :20], v[:, :20], beta[:, :20], decay[:, :20], s0, lib=lib)
        _close(od, o20, 1e-12, "dense")
        _close(sd, s20, 1e-12, "dense state")
    # tokens with a = 0 reset the state; strong decay (a ~ exp(-softplus(N(2,1))))
    q, k, v, beta, decay, s0 = rand_case(B=1, T=50, H=2, dk=8, dv=8, seed=20)
    decay[:, [0, 13, 14, 31], :] = 0.0
    rng = np.random.default_rng(21)
    decay[:, 40:, :] = np.exp(-np.logaddexp(0.0, rng.normal(2.0, 1.0, (1, 10, 2))))
    o, st = oracle.forward(q, k, v, beta, decay, s0, lib=lib)
    for C in (4, 16, 64):
        oc, sc = oracle.chunkwise(q, k, v, beta, decay, s0, chunk=C, lib=lib)
        _close(oc, o, 1e-12, f"chunkwise zero-decay C={C}")
        _close(sc, st, 1e-12, f"chunkwise zero-decay C={C} state")
    # with a = 0 at token 31, nothing before it reaches the state after it
    o2, _ = oracle.forward(q[:, 31:], k[:, 31:], v[:, 31:], beta[:, 31:], decay[:, 31:], None, lib=lib)
    _close(o2, o[:, 31:], 1e-13, "reset at a=0")


# -- (xiii) with unit keys and a, b in [0, 1]:  ||S_t|| <= a_t ||S_{t-1}|| + b_t ||v_t|| --
def pin_norm_bound(lib):
    q, k, v, beta, decay, s0 = rand_case(B=1, T=30, H=1, dk=8, dv=5, seed=22)
    s = s0
    for t in range(30):
        sl = slice(t, t + 1)
        _, s_new = oracle.forward(q[:, sl], k[:, sl], v[:, sl], beta[:, sl], decay[:, sl], s, lib=lib)
        bound = decay[0, t, 0] * np.linalg.norm(s) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(s_new) <= bound * (1 + 1e-12), t
        s = s_new


# -- hand-worked example (tests/golden/hand_d2_t3.txt) --------------------------------
def load_hand_example():
    toks, state = [], None
    with open(os.path.join(GOLDEN, "hand_d2_t3.txt")) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#"):
                continue
            if parts[0] == "token":
                toks.append([float(x) for x in parts[2:]])
            elif parts[0] == "state":
                state = np.array([float(x) for x in parts[1:]]).reshape(2, 2)
    a = np.array(toks)
    T = len(toks)
    k = a[:, 0:2].reshape(1, T, 1, 2)
    q = a[:, 2:4].reshape(1, T, 1, 2)
    v = a[:, 4:6].reshape(1, T, 1, 2)
    beta = a[:, 6].reshape(1, T, 1)
    decay = a[:, 7].reshape(1, T, 1)
    o_sqrt2 = a[:, 8:10]
    return q, k, v, beta, decay, o_sqrt2, state


def pin_hand_example(lib):
    q, k, v, beta, decay, o_sqrt2, state = load_hand_example()
    for fn in (oracle.forward, oracle.dense):
        out, st = fn(q, k, v, beta, decay, None, lib=lib)
        assert np.max(np.abs(out[0, :, 0] * np.sqrt(2.0) - o_sqrt2)) < 1e-12, fn.__name__
        assert np.max(np.abs(st[0, 0] - state)) < 1e-12, fn.__name__
    out, st = oracle.chunkwise(q, k, v, beta, decay, None, chunk=2, lib=lib)
    assert np.max(np.abs(out[0, :, 0] * np.sqrt(2.0) - o_sqrt2)) < 1e-12, "chunkwise"


ALL_PINS = [
    pin_zero_write_zero_state, pin_zero_write_decays_state, pin_single_token,
    pin_associative_recall, pin_decayed_recall, pin_single_key_ema, pin_lms_learns_linear_map,
    pin_linearity, pin_row_independence, pin_streaming_split, pin_bidi, pin_forms_agree,
    pin_norm_bound, pin_hand_example,
]
