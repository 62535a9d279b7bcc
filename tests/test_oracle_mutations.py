"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the oracle's pins catch every one of them."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_ref.py")

MUTATIONS = {
    "decay dropped": ("S = np.exp(g)[..., :, None] * S", "S = S"),
    "delta sign": ("(v - np.einsum(", "(v + np.einsum("),
    "output transposed": ('o = None if q_hat is None else np.einsum("...kv,...k->...v", S, q_hat)',
                          'o = None if q_hat is None else np.einsum("...kv,...v->...k", S, q_hat)'),
    "decay on the value axis": ("S = np.exp(g)[..., :, None] * S", "S = np.exp(g)[..., None, :] * S"),
    "eps outside the sqrt": ("np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)",
                             "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + L2_EPS)"),
    "scale on k": ("k_hat = l2_normalize(bf16_bits_to_f64(k_bits))",
                   "k_hat = l2_normalize(bf16_bits_to_f64(k_bits)) * float(np.float32(layer.scale))"),
    "beta not squashed": ("beta = sigmoid(bf16_bits_to_f64(b_bits))", "beta = bf16_bits_to_f64(b_bits)"),
    "A_log not exponentiated": ("a = np.exp(np.asarray(a_log, dtype=np.float64))",
                                "a = np.asarray(a_log, dtype=np.float64)"),
    "gate bias dropped": ("g = gate(bf16_bits_to_f64(g_bits) + g_bias, a_log, layer.lower_bound)",
                          "g = gate(bf16_bits_to_f64(g_bits), a_log, layer.lower_bound)"),
    "output before the update": (
        '    S = S + k_hat[..., :, None] * u[..., None, :]\n    o = None if q_hat is None else np.einsum("...kv,...k->...v", S, q_hat)',
        '    o = None if q_hat is None else np.einsum("...kv,...k->...v", S, q_hat)\n    S = S + k_hat[..., :, None] * u[..., None, :]'),
    "no window clamp": ("return min(max(int(n), 0), int(T), int(Q))", "return min(max(int(n), 0), int(T))"),
    "beta missing from the delta": ("u = beta[..., None] * (v - ", "u = (v - "),
    "final column one token late": ("col = min(max(c + n - 1, 0) // bs, width - 1)",
                                    "col = min(max(c + n, 0) // bs, width - 1)"),
    "final column not clamped": ("col = min(max(c + n - 1, 0) // bs, width - 1)",
                                 "col = max(c + n - 1, 0) // bs"),
    "boundary reached strictly": ("if c + n >= nb and bcol < width:", "if c + n > nb and bcol < width:"),
    "boundary length off by one": ("blen = nb - c\n", "blen = nb - c - 1\n"),
    "boundary column one block late": ("bcol = nb // bs - 1", "bcol = nb // bs"),
    "align replay restarts at 0": ("S = _replay(layer, S, rec, ri, n, start=blen)",
                                   "S = _replay(layer, S, rec, ri, n)"),
    "conv window one column late": ("vals = conv[src, :, n - 1:n - 1 + history].copy()",
                                    "vals = conv[src, :, n:n + history].copy()"),
    "conv boundary takes the final window": ("bvals = conv[src, :, blen - 1:blen - 1 + history].copy()",
                                             "bvals = conv[src, :, n - 1:n - 1 + history].copy()"),
    "spec source column not minus one": ("return min(max(int(num_accepted[i]), 1), int(cols)) - 1",
                                         "return min(max(int(num_accepted[i]), 1), int(cols) - 1)"),
    "spec state stored one column late": ("                dst = int(state_table[i, t])",
                                          "                dst = int(state_table[i, t + 1]) if t + 1 < cols else 0"),
    "spec null column stored": ("                if _slot_ok(dst, nslots):",
                                "                if dst < nslots:"),
    "spec state stored before the token": (
        "            S, out = kda_step(S, q_hat, k_hat, vv, gg, bb)\n            o[tok] = f64_to_bf16_bits(out)\n"
        "            if t < cols:\n                dst = int(state_table[i, t])\n"
        "                if _slot_ok(dst, nslots):\n                    _store_state(pool, dst, S)\n",
        "            if t < cols:\n                dst = int(state_table[i, t])\n"
        "                if _slot_ok(dst, nslots):\n                    _store_state(pool, dst, S)\n"
        "            S, out = kda_step(S, q_hat, k_hat, vv, gg, bb)\n            o[tok] = f64_to_bf16_bits(out)\n"),
    "align deferred commits every row": ("            if not now:\n                continue", "            pass"),
    "align deferred pending counts invalid rows": (
        "pending[ri - 1] = 0 if now else (n if (n > 0 and _slot_ok(src, nslots)) else 0)",
        "pending[ri - 1] = 0 if now else n"),
}

PIN_FILES = ("test_oracle.py", "test_oracle_commit_align.py", "test_oracle_spec.py")


def _run_pins(tmp_path, src):
    # A self-contained copy: the mutated oracle, the input generators, the
    # pins and their golden files.
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    (pkg / "kda_ref.py").write_text(src)
    shutil.copytree(os.path.join(ROOT, "workloads"), tmp_path / "workloads",
                    ignore=shutil.ignore_patterns("__pycache__"))
    tdir = tmp_path / "pins"
    tdir.mkdir()
    for f in PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", f), tdir / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tdir / "golden")
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "--rootdir", str(tmp_path), *[str(tdir / f) for f in PIN_FILES]],
                         cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    assert "passed" in res.stdout or "failed" in res.stdout, res.stdout[-2000:] + res.stderr[-2000:]
    return res


def test_unmodified_copy_passes(tmp_path):
    res = _run_pins(tmp_path, open(SRC).read())
    assert res.returncode == 0, res.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    a, b = MUTATIONS[name]
    assert a in src, f"mutation site for {name!r} not found"
    res = _run_pins(tmp_path, src.replace(a, b, 1))
    assert res.returncode != 0, f"the pins did not catch: {name}\n{res.stdout[-2000:]}"
