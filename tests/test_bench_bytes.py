"""The benchmark's byte accounting (CPU): the algorithmic bytes per call
follow the per-(row, head) counts of the method (state once or twice, each
token's inputs, output and records), and the counter data is keyed by the
kernel code without its comments."""

import importlib.util
import os

import numpy as np

from workloads import make_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench():
    spec = importlib.util.spec_from_file_location("kda_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_per_row_head_counts():
    b = bench()
    assert b.STATE_BYTES == 65536                      # 128 x 128 fp32
    assert b.TOKEN_IN_BYTES == 1026                    # q, k, v, g (128 bf16 each) + beta
    assert b.OUT_BYTES == 256 and b.REC_BYTES == 770   # o; records k, v, g + beta
    # one valid row, H = 1: verify of T tokens, commit of n
    v, c = b.algorithmic_bytes(np.array([4]), np.array([3]), np.array([True]), 1)
    assert v == 65536 + 2052 * 4
    assert c == 2 * 65536 + 770 * 3
    # nothing committed: no state traffic for the commit; skipped rows count nothing
    v, c = b.algorithmic_bytes(np.array([4, 2]), np.array([0, 2]), np.array([True, False]), 3)
    assert v == 3 * (65536 + 2052 * 4) and c == 0


def test_decode_workload_bytes():
    b = bench()
    batch = make_batch("decode")
    T = batch.seq_lens()
    n = np.minimum(np.maximum(batch.num_accepted, 0), np.minimum(T, batch.Q))
    v, c = b.algorithmic_bytes(T, n, batch.valid_rows(), batch.H)
    assert v == 64 * 32 * (65536 + 2052 * 4) == 151027712
    assert c == 32 * sum(2 * 65536 + 770 * int(k) for k in n if k > 0)


def test_deferred_bytes_fold_the_previous_count():
    b = bench()
    T, valid = np.array([4, 4]), np.array([True, True])
    n_prev, n_now = np.array([2, 0]), np.array([1, 3])
    no_eager = np.zeros(2, np.uint8)
    eager, vdef, cdef = b.deferred_bytes(T, n_prev, no_eager, n_now, no_eager, valid, 1)
    # the deferred verify reads every state, writes the folded one (row 0), reads 2 records
    assert vdef == 2 * (65536 + 2052 * 4) + 65536 + 770 * 2
    assert cdef == 0                                   # no eager row commits now
    assert eager == 2 * (65536 + 2052 * 4) + (2 * 65536 + 770) + (2 * 65536 + 770 * 3)


def test_counter_key_ignores_comments():
    b = bench()
    code = "int f(int x) {\n  return x + 1;  // one\n}\n"
    assert b.source_hash(code) == b.source_hash("/* header */\n" + code.replace("// one", "// two"))
    assert b.source_hash(code) != b.source_hash(code.replace("+ 1", "+ 2"))
