"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each test states what fixes the expected value: a hand-worked example, a
closed form, an invariant of the method, a special case with a textbook
answer, or a brute-force product form of the recurrence.
"""

import math
import os

import numpy as np
import pytest

from oracle import kda_ref as ref
from workloads import make_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 ----

def _f32_bits_to_bf16_exact(f32_bits):
    return np.uint16(f32_bits >> 16)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (mantissa 2)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just above the tie -> up
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),    # just below the tie -> down
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite bf16
    ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie between max and 2^128 -> inf
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # tie 0 / 2^-133 -> even (0)
    (1.5 * 2.0 ** -133, 0x0002),               # tie 1 / 2 quanta -> even (2)
    (2.0 ** -126, 0x0080),                     # smallest normal
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_bf16_rne_hand_picked(value, bits):
    # The bf16 format: sign, 8 exponent bits, 7 stored mantissa bits
    # (the top half of an IEEE binary32); ties round to the even mantissa.
    assert int(ref.f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = ref.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = ref.f64_to_bf16_bits(vals[finite])
    assert np.array_equal(back, bits[finite])
    assert np.all(np.isnan(vals[(bits & 0x7F80) == 0x7F80][(bits[(bits & 0x7F80) == 0x7F80] & 0x7F) != 0]))


def test_bf16_nearest_on_random_values():
    # Brute force: the nearest of all finite bf16 values (ties by even bits).
    rng = np.random.default_rng(7)
    x = rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 8, 2000)
    table_bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    table = ref.bf16_bits_to_f64(table_bits)
    got = ref.f64_to_bf16_bits(x)
    for xi, gi in zip(x, got):
        a = abs(xi)
        j = np.searchsorted(table, a)
        cands = [c for c in (j - 1, j) if 0 <= c < len(table)]
        dist = [abs(table[c] - a) for c in cands]
        best = min(dist)
        winners = [cands[i] for i, d in enumerate(dist) if d == best]
        w = winners[0] if len(winners) == 1 else [c for c in winners if c % 2 == 0][0]
        expect = int(table_bits[w]) | (0x8000 if xi < 0 else 0)
        assert int(gi) == expect


# ------------------------------------------------- elementary functions ----

def test_sigmoid_special_values():
    assert ref.sigmoid(np.array([0.0]))[0] == 0.5
    x = np.linspace(-40, 40, 81)
    assert np.allclose(ref.sigmoid(x) + ref.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert ref.sigmoid(np.array([-1000.0]))[0] == 0.0       # no overflow
    assert ref.sigmoid(np.array([1000.0]))[0] == 1.0
    assert ref.sigmoid(np.array([-np.inf]))[0] == 0.0
    for v in (-3.0, -0.5, 0.7, 4.0):                         # textbook scalar form
        assert math.isclose(ref.sigmoid(np.array([v]))[0], 1 / (1 + math.exp(-v)), rel_tol=1e-15)


def test_softplus_special_values():
    assert math.isclose(ref.softplus(np.array([0.0]))[0], math.log(2.0), rel_tol=1e-15)
    x = np.linspace(-30, 30, 61)
    # softplus(x) - softplus(-x) = x; softplus(x) -> x for large x, -> e^x for very negative x
    assert np.allclose(ref.softplus(x) - ref.softplus(-x), x, rtol=0, atol=1e-12)
    assert math.isclose(ref.softplus(np.array([50.0]))[0], 50.0, rel_tol=1e-15)
    assert math.isclose(ref.softplus(np.array([-50.0]))[0], math.exp(-50.0), rel_tol=1e-12)
    assert ref.softplus(np.array([800.0]))[0] == 800.0       # no overflow


def test_l2_normalize_unit_norm_and_eps_inside_sqrt():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128)) * 3
    y = ref.l2_normalize(x)
    n2 = np.sum(x * x, axis=-1)
    assert np.allclose(np.sum(y * y, axis=-1), n2 / (n2 + 1e-6), rtol=1e-14)
    assert np.allclose(y / np.linalg.norm(y, axis=-1, keepdims=True),
                       x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=1e-14)
    # The eps sits inside the square root: a vector with sum of squares 1e-6
    # comes out with norm 1/sqrt(2) (with eps outside it would be ~0.999).
    z = np.zeros(128)
    z[3] = 1e-3
    assert math.isclose(np.linalg.norm(ref.l2_normalize(z)), 2 ** -0.5, rel_tol=1e-12)


def test_gate_bounded_and_unbounded():
    x = np.linspace(-8, 8, 401)
    a_log = np.log(3.0)
    gb = ref.gate(x, a_log, -5.0)
    assert np.all(gb > -5.0) and np.all(gb < 0.0)
    assert np.all(ref.gate(np.array([-300.0, 300.0]), a_log, -5.0) >= -5.0)
    assert ref.gate(np.array([0.0]), a_log, -5.0)[0] == -2.5      # lb * sigmoid(0)
    assert np.all(np.diff(gb) < 0)                                  # more x, more decay
    gu = ref.gate(x, a_log, None)
    assert np.all(gu <= 0.0)
    assert math.isclose(ref.gate(np.array([0.0]), a_log, None)[0], -3.0 * math.log(2.0), rel_tol=1e-15)
    assert math.isclose(ref.gate(np.array([40.0]), a_log, None)[0], -120.0, rel_tol=1e-15)
    # lower bound 0 closes the gate: g = 0 exactly (used by the memory pin below)
    assert np.all(ref.gate(x, a_log, 0.0) == 0.0)


# ------------------------------------------------------------ the step ----

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = np.array([float(t) for t in rest])
    return vals


def test_step_hand_worked_example():
    gv = _read_golden("hand_step_2x2.txt")
    S0 = gv["S0"].reshape(2, 2)
    S1, o = ref.kda_step(S0, gv["q_hat"], gv["k_hat"], gv["v"], gv["g"], gv["beta"][0])
    assert np.allclose(S1, gv["S1"].reshape(2, 2), rtol=0, atol=1e-15)
    assert np.allclose(o, gv["o"], rtol=0, atol=1e-15)


def test_step_delta_rule_closed_form():
    # g = 0, beta = 1, unit key: after the step S'^T k = v for any S.
    rng = np.random.default_rng(2)
    for K, V in ((3, 5), (8, 4), (128, 128)):
        S = rng.standard_normal((K, V))
        k = rng.standard_normal(K)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(V)
        S1, _ = ref.kda_step(S, None, k, v, np.zeros(K), np.float64(1.0))
        assert np.allclose(S1.T @ k, v, rtol=0, atol=1e-12)


def test_step_orthonormal_memory():
    # g = 0, beta = 1, S0 = 0, orthonormal keys: every stored value is recalled.
    rng = np.random.default_rng(3)
    K, V, n = 16, 6, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys, vals = Qm[:, :n].T, rng.standard_normal((n, V))
    S = np.zeros((K, V))
    for j in range(n):
        S, _ = ref.kda_step(S, None, keys[j], vals[j], np.zeros(K), np.float64(1.0))
    for j in range(n):
        assert np.allclose(S.T @ keys[j], vals[j], rtol=0, atol=1e-12)


def test_step_pure_decay_per_key_channel():
    # beta = 0: S_n = diag(exp(sum_t g_t)) S0; the decay acts on key channels (rows).
    rng = np.random.default_rng(4)
    K, V = 5, 7
    S0 = rng.standard_normal((K, V))
    S, gs = S0.copy(), np.zeros(K)
    for _ in range(4):
        g = -rng.random(K) * 2
        gs += g
        S, _ = ref.kda_step(S, rng.standard_normal(K), rng.standard_normal(K),
                            rng.standard_normal(V), g, np.float64(0.0))
    assert np.allclose(S, np.exp(gs)[:, None] * S0, rtol=1e-13, atol=0)
    # g -> -inf wipes the state
    S1, _ = ref.kda_step(S0, None, np.ones(K), np.zeros(V), np.full(K, -np.inf), np.float64(0.0))
    assert np.all(S1 == 0.0)


def _product_form(S0, qh, kh, v, g, beta):
    """S_n = P_n...P_1 S0 + sum_t P_n...P_{t+1} beta_t k_t v_t^T with
    P_t = (I - beta_t k_t k_t^T) diag(exp g_t); o_t = S_t^T q_t, all as dense
    matrix products."""
    K = S0.shape[0]
    T = len(kh)
    P = [(np.eye(K) - beta[t] * np.outer(kh[t], kh[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    outs, states = [], []
    for n in range(1, T + 1):
        M = np.eye(K)
        for t in range(n):
            M = P[t] @ M
        Sn = M @ S0
        for t in range(n):
            L = np.eye(K)
            for s in range(t + 1, n):
                L = P[s] @ L
            Sn = Sn + L @ (beta[t] * np.outer(kh[t], v[t]))
        states.append(Sn)
        outs.append(Sn.T @ qh[n - 1])
    return states, outs


@pytest.mark.parametrize("K,V,T", [(2, 3, 4), (4, 4, 3), (8, 2, 4), (8, 8, 1)])
def test_step_matches_brute_force_product_form(K, V, T):
    rng = np.random.default_rng(K * 100 + V * 10 + T)
    S0 = rng.standard_normal((K, V))
    qh = rng.standard_normal((T, K))
    kh = ref.l2_normalize(rng.standard_normal((T, K)))
    v = rng.standard_normal((T, V))
    g = -rng.random((T, K)) * 3
    beta = rng.random(T)
    states, outs = _product_form(S0, qh, kh, v, g, beta)
    S = S0
    for t in range(T):
        S, o = ref.kda_step(S, qh[t], kh[t], v[t], g[t], beta[t])
        assert np.allclose(S, states[t], rtol=1e-12, atol=1e-12)
        assert np.allclose(o, outs[t], rtol=1e-12, atol=1e-12)


# ------------------------------------------------ the pipeline (calls) ----

def _bits(x):
    return ref.f64_to_bf16_bits(np.asarray(x, np.float64))


def _tiny_pipeline(K=4, H=2, T=3, seed=5, lower_bound=-5.0):
    rng = np.random.default_rng(seed)
    layer = ref.Layer(a_log=np.log(rng.uniform(1, 16, H)).astype(np.float32),
                      g_bias=(rng.standard_normal(H * K) * 0.1).astype(np.float32),
                      scale=float(np.float32(K ** -0.5)), lower_bound=lower_bound)
    q, k, v, g = (_bits(rng.standard_normal((T, H, K))) for _ in range(4))
    beta = _bits(rng.standard_normal((T, H)))
    pool = (rng.standard_normal((2, H, K, K)) * 0.3).astype(np.float32)
    return layer, q, k, v, g, beta, pool


@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_recurrent_matches_product_form_from_raw_inputs(lower_bound):
    # The whole call against the dense product form built from the page's
    # definitions of q^, k^, g and beta (scale on q only, eps inside the sqrt).
    K, H, T = 4, 2, 3
    layer, q, k, v, g, beta, pool = _tiny_pipeline(K, H, T, lower_bound=lower_bound)
    pool0 = pool.copy()
    o = np.zeros((T, H, K), np.uint16)
    ref.kda_recurrent(layer, q, k, v, g, beta, np.array([0, T], np.int32), pool,
                      np.array([1], np.int32), o)
    f = ref.bf16_bits_to_f64
    for h in range(H):
        qh = np.stack([f(q[t, h]) / math.sqrt(np.sum(f(q[t, h]) ** 2) + 1e-6)
                       * float(np.float32(layer.scale)) for t in range(T)])
        kh = np.stack([f(k[t, h]) / math.sqrt(np.sum(f(k[t, h]) ** 2) + 1e-6) for t in range(T)])
        x = f(g[:, h]) + layer.g_bias.reshape(H, K)[h].astype(np.float64)
        A = math.exp(float(layer.a_log[h]))
        if lower_bound is None:
            gg = -A * np.log1p(np.exp(x))
        else:
            gg = lower_bound / (1 + np.exp(-A * x))
        bb = 1 / (1 + np.exp(-f(beta[:, h])))
        states, outs = _product_form(pool0[1, h].astype(np.float64).T, qh, kh, f(v[:, h]), gg, bb)
        assert np.allclose(pool[1, h].T, states[-1], rtol=1e-6, atol=1e-7)
        for t in range(T):
            assert np.array_equal(o[t, h], ref.f64_to_bf16_bits(outs[t]))
    assert np.array_equal(pool[0], pool0[0])          # other slot untouched


def test_recurrent_orthonormal_keys_recall_values():
    # g = 0 (lower bound 0), beta ~ 1 (beta_raw = 40), zero state, basis keys:
    # S_n^T e_j returns v_j up to the 1e-6 eps of the normalisation.
    K, H, n = 128, 2, 6
    layer = ref.Layer(a_log=np.zeros(H, np.float32), g_bias=np.zeros(H * K, np.float32),
                      scale=float(np.float32(K ** -0.5)), lower_bound=0.0)
    rng = np.random.default_rng(6)
    k = np.zeros((n, H, K))
    for j in range(n):
        k[j, :, 10 * j] = 1.0
    k = _bits(k)
    v = _bits(rng.standard_normal((n, H, K)))
    q = _bits(rng.standard_normal((n, H, K)))
    g = _bits(rng.standard_normal((n, H, K)))
    beta = _bits(np.full((n, H), 40.0))
    pool = np.zeros((2, H, K, K), np.float32)
    o = np.zeros((n, H, K), np.uint16)
    ref.kda_recurrent(layer, q, k, v, g, beta, np.array([0, n], np.int32), pool,
                      np.array([1], np.int32), o)
    S = pool[1].astype(np.float64).transpose(0, 2, 1)     # [H, K, V]
    for j in range(n):
        recall = S[:, 10 * j, :]                          # S^T e_j
        assert np.allclose(recall, ref.bf16_bits_to_f64(v[j]), rtol=3e-6, atol=1e-7)


def test_recurrent_pure_decay_from_raw_inputs():
    # beta_raw = -inf gives beta = 0: the state only decays, per key channel.
    K, H, T = 128, 2, 3
    layer, q, k, v, g, beta, pool = _tiny_pipeline(K, H, T, lower_bound=None)
    beta[:] = 0xFF80
    pool0 = pool.copy()
    o = np.zeros((T, H, K), np.uint16)
    ref.kda_recurrent(layer, q, k, v, g, beta, np.array([0, T], np.int32), pool,
                      np.array([1], np.int32), o)
    f = ref.bf16_bits_to_f64
    for h in range(H):
        x = f(g[:, h]) + layer.g_bias.reshape(H, K)[h]
        gsum = np.sum(-math.exp(float(layer.a_log[h])) * np.log1p(np.exp(x)), axis=0)
        expect = pool0[1, h].astype(np.float64) * np.exp(gsum)[None, :]   # stored [V, K]
        assert np.allclose(pool[1, h], expect, rtol=1e-6, atol=1e-30)


# ------------------------------------------------ RecoverSSM invariants ----

def _oracle_inputs(name="tiny", **kw):
    b = make_batch(name, **kw)
    layer = ref.Layer(b.a_log, b.g_bias, b.scale, b.lower_bound)
    t = b.tokens
    return b, layer, (t.q, t.k, t.v, t.g, t.beta)


def test_verify_leaves_pool_and_records_raw_inputs():
    b, layer, toks = _oracle_inputs()
    pool = b.initial_pool()
    pool0 = pool.copy()
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K, fill=0xABCD)
    o = np.zeros((toks[0].shape[0], b.H, b.K), np.uint16)
    ref.kda_verify(layer, *toks, b.cu_seqlens, pool, b.state_indices, rec, o)
    assert np.array_equal(pool, pool0)
    q, k, v, g, beta = toks
    for i in range(b.num_rows):
        bos, T = int(b.cu_seqlens[i]), int(b.seq_lens()[i])
        assert np.array_equal(rec.k[i + 1, :, :T], k[bos:bos + T].transpose(1, 0, 2))
        assert np.array_equal(rec.v[i + 1, :, :T], v[bos:bos + T].transpose(1, 0, 2))
        assert np.array_equal(rec.g[i + 1, :, :T], g[bos:bos + T].transpose(1, 0, 2))
        assert np.array_equal(rec.beta[i + 1, :, :T], beta[bos:bos + T].T)
    assert np.all(rec.k[0] == 0xABCD)           # scratch row untouched


def test_verify_outputs_equal_recurrent_outputs():
    b, layer, toks = _oracle_inputs()
    o1 = np.zeros((toks[0].shape[0], b.H, b.K), np.uint16)
    o2 = o1.copy()
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K)
    ref.kda_verify(layer, *toks, b.cu_seqlens, b.initial_pool(), b.state_indices, rec, o1)
    ref.kda_recurrent(layer, *toks, b.cu_seqlens, b.initial_pool(), b.state_indices, o2)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("n_override", [None, 0, -3, 7])
def test_commit_equals_recurrence_over_accepted_prefix(n_override):
    b, layer, toks = _oracle_inputs()
    q, k, v, g, beta = toks
    ntok = q.shape[0]
    nacc = b.num_accepted.copy() if n_override is None else np.full(b.num_rows, n_override, np.int32)
    pool = b.initial_pool()
    pool0 = pool.copy()
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K)
    o = np.zeros((ntok, b.H, b.K), np.uint16)
    ref.kda_verify(layer, *toks, b.cu_seqlens, pool, b.state_indices, rec, o)
    ref.kda_commit(layer, b.cu_seqlens, ntok, pool, b.state_indices, rec, nacc)
    for i in range(b.num_rows):
        slot = b.state_indices[i]
        T = int(b.seq_lens()[i])
        n = min(max(int(nacc[i]), 0), T, b.Q)
        if n == 0:
            assert np.array_equal(pool[slot], pool0[slot])       # untouched, bitwise
            continue
        # the state after the first n tokens, by the plain recurrence
        pr = pool0.copy()
        cu = np.array([0, n], np.int32)
        bos = int(b.cu_seqlens[i])
        sl = slice(bos, bos + n)
        ref.kda_recurrent(layer, q[sl], k[sl], v[sl], g[sl], beta[sl], cu, pr,
                          np.array([slot], np.int32), np.zeros((n, b.H, b.K), np.uint16))
        assert np.array_equal(pool[slot], pr[slot])


def test_skipped_rows_touch_nothing():
    b, layer, toks = _oracle_inputs("ragged", B=12, H=2)
    q = toks[0]
    ntok = q.shape[0]
    pool = b.initial_pool()
    pool0 = pool.copy()
    o = np.full((ntok, b.H, b.K), 0x7E7E, np.uint16)
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K, fill=0x1234)
    si = b.state_indices.copy()
    si[[0, 3]] = [0, -1]
    ref.kda_verify(layer, *toks, b.cu_seqlens, pool, si, rec, o)
    for i in (0, 3):
        bos, T = int(b.cu_seqlens[i]), int(b.seq_lens()[i])
        assert np.all(o[bos:bos + T] == 0x7E7E)
        assert np.all(rec.k[i + 1] == 0x1234)
    ref.kda_commit(layer, b.cu_seqlens, ntok, pool, si, rec, np.full(b.num_rows, 8, np.int32))
    assert np.array_equal(pool[0], pool0[0])


def test_deferred_flow_equals_eager_flow():
    # Two steps of verify -> commit. Eager: commit at once. Deferred: commit
    # turns n' into pending (except eager rows), the next verify folds it,
    # and a final flush (verify with no tokens) folds the rest.
    H, B = 2, 6
    b0, layer, t0 = _oracle_inputs("tiny", B=B, H=H)
    b1, _, t1 = _oracle_inputs("ragged", B=B, H=H)
    Q = 4
    t1 = tuple(x[:B * Q] for x in t1)
    cu1 = (np.arange(B + 1) * Q).astype(np.int32)
    steps = [(t0, b0.cu_seqlens), (t1, cu1)]
    nacc = [np.array([0, 1, 2, 3, 4, 9], np.int32), np.array([4, 3, 0, 2, 1, 4], np.int32)]
    eager = [np.array([0, 1, 0, 0, 1, 0], np.uint8), np.array([0, 0, 1, 0, 0, 0], np.uint8)]
    rr = np.array([3, 0, 5, 1, 4, 2], np.int32)
    si = b0.state_indices
    pool_e, pool_d = b0.initial_pool(), b0.initial_pool()
    ntok = t0[0].shape[0]
    # eager
    oe = []
    for (toks, cu), n in zip(steps, nacc):
        o = np.zeros((ntok, H, 128), np.uint16)
        rec = ref.Records.empty(B, H, Q, 128)
        ref.kda_verify(layer, *toks, cu, pool_e, si, rec, o, record_rows=rr)
        ref.kda_commit(layer, cu, ntok, pool_e, si, rec, n, record_rows=rr)
        oe.append(o)
    # deferred
    pending = np.zeros(B, np.int32)
    recs = [ref.Records.empty(B, H, Q, 128), ref.Records.empty(B, H, Q, 128)]
    for s, ((toks, cu), n) in enumerate(zip(steps, nacc)):
        o = np.zeros((ntok, H, 128), np.uint16)
        ref.kda_verify_deferred(layer, *toks, cu, pool_d, si, recs[(s + 1) % 2], pending,
                                recs[s % 2], rr, o)
        assert np.array_equal(o, oe[s])
        ref.kda_commit(layer, cu, ntok, pool_d, si, recs[s % 2], n, record_rows=rr,
                       pending=pending, eager=eager[s])
        for i in range(B):
            nn = min(max(int(n[i]), 0), Q)
            assert pending[rr[i]] == (0 if eager[s][i] else nn)
    empty_cu = np.zeros(B + 1, np.int32)
    ref.kda_verify_deferred(layer, *t0, empty_cu, pool_d, si, recs[1], pending, recs[0], rr,
                            np.zeros((ntok, H, 128), np.uint16))
    assert np.array_equal(pool_d, pool_e)


def test_commit_clamps_to_the_record_window():
    # A row longer than the window Q records only Q tokens, and commit(n)
    # replays at most Q of them (n' = min(max(n, 0), T_i, Q)).
    b, layer, toks = _oracle_inputs("ragged", B=16, H=2)
    q, k, v, g, beta = toks
    ntok = q.shape[0]
    T = b.seq_lens()
    i = int(np.argmax(T))
    assert T[i] > 4
    cu = b.cu_seqlens
    Q = 4
    si = np.zeros(b.num_rows, np.int32)
    si[i] = b.state_indices[i] if b.state_indices[i] > 0 else 7
    pool = b.initial_pool()
    pool[si[i]] = np.float32(0.01)
    pool0 = pool.copy()
    rec = ref.Records.empty(b.num_rows, b.H, Q, b.K, fill=0x5555)
    ref.kda_verify(layer, *toks, cu, pool, si, rec, np.zeros((ntok, b.H, b.K), np.uint16))
    bos = int(cu[i])
    assert np.array_equal(rec.k[i + 1], k[bos:bos + Q].transpose(1, 0, 2))
    ref.kda_commit(layer, cu, ntok, pool, si, rec, np.full(b.num_rows, 8, np.int32))
    pr = pool0.copy()
    sl = slice(bos, bos + Q)
    ref.kda_recurrent(layer, q[sl], k[sl], v[sl], g[sl], beta[sl], np.array([0, Q], np.int32),
                      pr, np.array([si[i]], np.int32), np.zeros((Q, b.H, b.K), np.uint16))
    assert np.array_equal(pool[si[i]], pr[si[i]])
