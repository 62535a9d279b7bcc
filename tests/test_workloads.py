"""The seeded synthetic workloads: deterministic, with the shapes, slot rules
and value distributions their recipe states (CPU only)."""

import numpy as np
import pytest

from workloads import CONFIG_NAMES, make_batch, make_deferred
from workloads.configs import bf16_to_f32, checkpoint_slot

SINGLE = ("tiny", "decode", "deep", "ragged")


def _small(name):
    # every recipe rule is the same at a reduced batch; the value statistics
    # below use the full head count of each recipe
    return make_batch(name, B={"tiny": None, "decode": 16, "deep": 32, "ragged": 64}[name])


def test_config_names():
    assert set(CONFIG_NAMES) == set(SINGLE) | {"deferred"}


@pytest.mark.parametrize("name", SINGLE)
def test_single_call_workloads_are_deterministic(name):
    a, b = _small(name), _small(name)
    for x, y in ((a.tokens.qkv, b.tokens.qkv), (a.tokens.g, b.tokens.g), (a.tokens.beta, b.tokens.beta),
                 (a.cu_seqlens, b.cu_seqlens), (a.state_indices, b.state_indices),
                 (a.num_accepted, b.num_accepted), (a.a_log, b.a_log), (a.g_bias, b.g_bias)):
        assert np.array_equal(x, y)
    assert np.array_equal(a.initial_pool(), b.initial_pool())


@pytest.mark.parametrize("name", SINGLE)
def test_shapes_slots_and_counts(name):
    b = _small(name)
    B, H, K = b.num_rows, b.H, b.K
    T = b.seq_lens()
    assert b.cu_seqlens[0] == 0 and np.all(np.diff(b.cu_seqlens) == T)
    assert b.tokens.qkv.shape == (int(T.sum()), 3 * H * K)
    assert b.tokens.g.shape == (int(T.sum()), H, K) and b.tokens.beta.shape == (int(T.sum()), H)
    assert np.all(T >= 1) and np.all(T <= b.Q)
    used = b.state_indices[b.state_indices > 0]
    assert len(np.unique(used)) == len(used), "distinct rows use distinct slots"
    assert np.all(used < b.num_slots)
    n = b.num_accepted
    assert np.all(n >= 0) and np.all(n <= T)
    assert b.a_log.dtype == np.float32 and b.a_log.shape == (H,)
    assert np.all((np.exp(b.a_log) >= 1.0) & (np.exp(b.a_log) <= 16.0))
    assert b.g_bias.shape == (H * K,)


def test_recipe_specifics():
    tiny = make_batch("tiny")
    assert (tiny.num_rows, tiny.H, tiny.Q) == (4, 4, 4)
    assert np.array_equal(tiny.state_indices, [1, 2, 3, 4]) and not tiny.g_bias.any()
    assert tiny.lower_bound is None
    dec = make_batch("decode", B=8)
    assert dec.init == "prefill" and dec.prefill.num_tokens == 8 * 64
    assert np.array_equal(dec.state_indices, np.arange(1, 9))
    assert not dec.initial_pool().any()           # the checkpoints come from the prefill
    rag = make_batch("ragged")
    skipped = rag.state_indices <= 0
    assert 0.02 < skipped.mean() < 0.2            # 10% of the rows, skipped by slot 0 or -1
    assert set(np.unique(rag.state_indices[skipped])) <= {0, -1}
    assert rag.lower_bound == -5.0 and rag.Q == 8
    assert set(np.unique(rag.seq_lens())) <= set(range(1, 9)) and len(np.unique(rag.seq_lens())) > 4


def test_value_distributions():
    b = make_batch("ragged", B=64)
    x = bf16_to_f32(b.tokens.qkv).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    g = bf16_to_f32(b.tokens.g).astype(np.float64)
    assert abs(g.std() - 2.0) < 0.02                      # ragged's g_raw ~ N(0, 2)
    assert abs(b.g_bias.std() - 0.1) < 0.01
    s = checkpoint_slot(b.seed, 0, 5, 4)
    assert s.dtype == np.float32 and s.shape == (4, 128, 128)
    assert abs(s.std() - 0.02) < 0.001
    # bf16 patterns are exact roundings: widening and rounding again is the identity
    from workloads.configs import bf16_from_f32
    assert np.array_equal(bf16_from_f32(bf16_to_f32(b.tokens.beta)), b.tokens.beta)


def test_deferred_run():
    r = make_deferred(B=32, H=4, layers=3)
    assert (r.T, r.Q, r.num_slots) == (4, 4, 33)
    assert np.array_equal(np.sort(r.state_indices), np.arange(1, 33))
    assert np.array_equal(np.sort(r.record_rows), np.arange(32))
    for s in range(r.steps):
        n = r.num_accepted(s)
        assert np.all((n >= 0) & (n <= r.T))
        assert np.array_equal(n, r.num_accepted(s))        # deterministic per step
    e = np.concatenate([r.eager(s) for s in range(r.steps)])
    assert set(np.unique(e)) <= {0, 1} and 0.05 < e.mean() < 0.4
    assert not np.array_equal(r.tokens(0, 0).qkv, r.tokens(1, 0).qkv)   # per layer
    assert not np.array_equal(r.tokens(0, 0).qkv, r.tokens(0, 1).qkv)   # per step
    assert np.array_equal(r.tokens(2, 1).g, r.tokens(2, 1).g)
    assert not np.array_equal(r.params[0].a_log, r.params[1].a_log)
