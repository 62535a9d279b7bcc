"""CPU checks of the C ABI: the library loads, exports every call that
include/kda.h declares, and rejects bad arguments on the host before anything
is enqueued (no GPU needed: the pointers below are never dereferenced)."""

import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_speculative_kda_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libkda.so not built")

E = {name: code for code, name in _lib.STATUS_NAMES.items()}
A = 0x10000000  # fake, aligned device addresses (never dereferenced on the host)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for name in ("kda_recurrent", "kda_verify", "kda_commit", "kda_verify_deferred",
                 "kda_status_string"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    lib = _lib.load()
    for f in declared_functions():
        assert hasattr(lib, f)


def test_status_strings():
    for code, name in _lib.STATUS_NAMES.items():
        assert _lib.status_string(code).startswith(name)
    assert "unknown" in _lib.status_string(99)


# ------------------------------------------------------------ validation --

H, K = 4, 128


def layer(**kw):
    d = dict(num_heads=H, head_dim=K, scale=K ** -0.5, has_lower_bound=0, lower_bound=0.0,
             a_log=A, g_bias=A + 0x1000)
    d.update(kw)
    return _lib.KdaLayer(**d)


def tokens(n_tok=8, n_rows=2, **kw):
    hk = H * K
    d = dict(q=A + 0x100000, k=A + 0x100000 + 2 * hk, v=A + 0x100000 + 4 * hk,
             g=A + 0x200000, beta=A + 0x300000, stride_q=3 * hk, stride_k=3 * hk,
             stride_v=3 * hk, stride_g=hk, stride_beta=H, cu_seqlens=A + 0x400000,
             num_rows=n_rows, num_tokens=n_tok)
    d.update(kw)
    return _lib.KdaTokens(**d)


def pool(**kw):
    d = dict(state=A + 0x1000000, slot_stride=H * K * K, num_slots=5, state_indices=A + 0x500000)
    d.update(kw)
    return _lib.KdaPool(**d)


def records(base=A + 0x8000000, rows=4, window=4, **kw):
    per = (rows + 1) * H * window * K * 2
    d = dict(k=base, v=base + per, g=base + 2 * per, beta=base + 3 * per, rows=rows, window=window)
    d.update(kw)
    return _lib.KdaRecords(**d)


O = A + 0x4000000   # an output range away from everything else


def verify(L=None, T=None, P=None, R=None, rr=None, o=O):
    lib = _lib.load()
    return lib.kda_verify(ctypes.byref(L or layer()), ctypes.byref(T or tokens()),
                          ctypes.byref(P or pool()), ctypes.byref(R or records()), rr, o, None)


def test_verify_rejects_bad_layer():
    lib = _lib.load()
    assert lib.kda_verify(None, ctypes.byref(tokens()), ctypes.byref(pool()),
                          ctypes.byref(records()), None, O, None) == E["KDA_ERR_NULL"]
    assert verify(L=layer(head_dim=64)) == E["KDA_ERR_UNSUPPORTED"]
    assert verify(L=layer(num_heads=0)) == E["KDA_ERR_SHAPE"]
    assert verify(L=layer(a_log=0)) == E["KDA_ERR_NULL"]


def test_verify_rejects_bad_tokens():
    assert verify(T=tokens(q=0)) == E["KDA_ERR_NULL"]
    assert verify(T=tokens(stride_q=100)) == E["KDA_ERR_SHAPE"]           # < H*K
    assert verify(T=tokens(stride_g=H * K + 2)) == E["KDA_ERR_ALIGN"]     # not a multiple of 4
    assert verify(T=tokens(k=A + 0x100000 + 2 * H * K + 2)) == E["KDA_ERR_ALIGN"]
    assert verify(T=tokens(num_rows=-1)) == E["KDA_ERR_SHAPE"]
    assert verify(T=tokens(max_seqlen=-1)) == E["KDA_ERR_SHAPE"]


def test_verify_rejects_bad_pool_and_records():
    assert verify(P=pool(state=A + 0x1000004)) == E["KDA_ERR_ALIGN"]
    assert verify(P=pool(slot_stride=H * K * K - 4)) == E["KDA_ERR_SHAPE"]
    assert verify(P=pool(slot_stride=H * K * K + 2)) == E["KDA_ERR_ALIGN"]
    assert verify(R=records(window=0)) == E["KDA_ERR_SHAPE"]
    assert verify(R=records(window=65)) == E["KDA_ERR_SHAPE"]
    assert verify(R=records(k=0)) == E["KDA_ERR_NULL"]
    # identity record rows need num_rows <= rows
    assert verify(T=tokens(n_rows=5), R=records(rows=4)) == E["KDA_ERR_CAPACITY"]


def test_verify_rejects_aliasing():
    # o overlapping the token arrays, the pool or the records
    assert verify(o=A + 0x100000 + 64) == E["KDA_ERR_ALIAS"]
    assert verify(o=A + 0x1000000 + 1024) == E["KDA_ERR_ALIAS"]
    assert verify(o=A + 0x8000000 + 2) == E["KDA_ERR_ALIAS"]
    # records overlapping each other
    r = records()
    r.v = r.k + 64
    assert verify(R=r) == E["KDA_ERR_ALIAS"]


def spec(L=None, T=None, P=None, tab=None, o=O, null_table=False):
    lib = _lib.load()
    if tab is None:
        tab = _lib.KdaSpecTable(indices=A + 0x600000, row_stride=4, cols=4, num_accepted=A + 0x700000)
    return lib.kda_recurrent_spec(ctypes.byref(L or layer()), ctypes.byref(T or tokens()),
                                  ctypes.byref(P or pool(state_indices=None)),
                                  None if null_table else ctypes.byref(tab), o, None)


def test_recurrent_spec_validation():
    assert spec(null_table=True) == E["KDA_ERR_NULL"]
    assert spec(tab=_lib.KdaSpecTable(indices=A, row_stride=4, cols=0)) == E["KDA_ERR_SHAPE"]
    assert spec(tab=_lib.KdaSpecTable(indices=A, row_stride=3, cols=4)) == E["KDA_ERR_SHAPE"]
    assert spec(tab=_lib.KdaSpecTable(indices=0, row_stride=4, cols=4)) == E["KDA_ERR_NULL"]
    assert spec(L=layer(head_dim=64)) == E["KDA_ERR_UNSUPPORTED"]
    assert spec(T=tokens(q=0)) == E["KDA_ERR_NULL"]
    assert spec(P=pool(state=A + 0x1000004, state_indices=None)) == E["KDA_ERR_ALIGN"]
    assert spec(o=0) == E["KDA_ERR_NULL"]
    assert spec(o=A + 0x1000000 + 1024) == E["KDA_ERR_ALIAS"]     # o inside the pool
    assert spec(o=A + 0x100000 + 64) == E["KDA_ERR_ALIAS"]        # o inside the tokens
    # the block ids or the counts inside the pool or o (both are written)
    assert spec(tab=_lib.KdaSpecTable(indices=A + 0x1000000 + 4096, row_stride=4, cols=4,
                                      num_accepted=A + 0x700000)) == E["KDA_ERR_ALIAS"]
    assert spec(tab=_lib.KdaSpecTable(indices=A + 0x600000, row_stride=4, cols=4,
                                      num_accepted=O + 16)) == E["KDA_ERR_ALIAS"]
    # a token array inside the pool
    assert spec(T=tokens(q=A + 0x1000000 + 8192)) == E["KDA_ERR_ALIAS"]
    # no rows: nothing to do, even without a table array
    assert spec(T=tokens(n_rows=0, num_tokens=0),
                tab=_lib.KdaSpecTable(indices=0, row_stride=4, cols=4)) == E["KDA_OK"]


def test_recurrent_alias():
    lib = _lib.load()
    rec = lambda T, o=O: lib.kda_recurrent(ctypes.byref(layer()), ctypes.byref(T),  # noqa: E731
                                           ctypes.byref(pool()), o, None)
    assert rec(tokens(), o=A + 0x1000000 + 1024) == E["KDA_ERR_ALIAS"]   # o inside the pool
    assert rec(tokens(g=A + 0x1000000 + 8192)) == E["KDA_ERR_ALIAS"]     # g inside the pool


def test_empty_batch_is_a_no_op():
    # num_rows == 0 returns OK before anything is enqueued (no GPU touched)
    assert verify(T=tokens(n_rows=0, num_tokens=0)) == E["KDA_OK"]
    lib = _lib.load()
    assert lib.kda_recurrent(ctypes.byref(layer()), ctypes.byref(tokens(n_rows=0)),
                             ctypes.byref(pool()), O, None) == E["KDA_OK"]
    assert lib.kda_commit(ctypes.byref(layer()), A, 0, ctypes.byref(pool()),
                          ctypes.byref(records()), None, A, None, None, None) == E["KDA_OK"]
    # per-row arrays may be NULL when there are no rows
    assert verify(T=tokens(n_rows=0, num_tokens=0), P=pool(state_indices=0)) == E["KDA_OK"]
    assert lib.kda_commit(ctypes.byref(layer()), A, 0, ctypes.byref(pool(state_indices=0)),
                          ctypes.byref(records()), None, None, None, None, None) == E["KDA_OK"]


def test_commit_validation():
    lib = _lib.load()
    c = lambda **kw: lib.kda_commit(  # noqa: E731
        ctypes.byref(kw.get("L", layer())), kw.get("cu", A), kw.get("n", 2),
        ctypes.byref(kw.get("P", pool())), ctypes.byref(kw.get("R", records())),
        kw.get("rr"), kw.get("acc", A + 0x600000), kw.get("pending"), kw.get("eager"), None)
    assert c(cu=0) == E["KDA_ERR_NULL"]
    assert c(acc=0) == E["KDA_ERR_NULL"]
    assert c(n=-1) == E["KDA_ERR_SHAPE"]
    assert c(eager=A + 0x700000) == E["KDA_ERR_SHAPE"]               # eager without pending
    assert c(n=5, R=records(rows=4)) == E["KDA_ERR_CAPACITY"]
    assert c(R=records(base=A + 0x1000000)) == E["KDA_ERR_ALIAS"]    # records inside the pool
    assert c(pending=A + 0x1000000) == E["KDA_ERR_ALIAS"]            # pending inside the pool


def test_verify_deferred_validation():
    lib = _lib.load()

    def d(rp=None, rn=None, pending=A + 0x700000, o=O):
        return lib.kda_verify_deferred(ctypes.byref(layer()), ctypes.byref(tokens()),
                                       ctypes.byref(pool()), ctypes.byref(rp or records()),
                                       pending, ctypes.byref(rn or records(base=A + 0xC000000)),
                                       None, o, None)
    assert d(pending=0) == E["KDA_ERR_NULL"]
    assert d(rn=records()) == E["KDA_ERR_ALIAS"]                       # rec_prev == rec_next
    assert d(rn=records(base=A + 0xC000000, window=8)) == E["KDA_ERR_SHAPE"]
    assert d(rn=records(base=A + 0xC000000, rows=3)) == E["KDA_ERR_SHAPE"]
    assert d(pending=A + 0xC000000) == E["KDA_ERR_ALIAS"]              # pending inside rec_next
    assert d(o=A + 0xC000000) == E["KDA_ERR_ALIAS"]


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


# ------------------------------------------------------------ multi-layer --

def layer_arrays(n=3, over=None):
    """n layers, each with its own pool and records, far apart; `over` maps a
    layer index to field overrides: {"layer": {...}, "pool": {...}, "rec": {...}}."""
    over = over or {}
    Ls, Ps, Rs = [], [], []
    for l in range(n):
        o = over.get(l, {})
        Ls.append(layer(**o.get("layer", {})))
        Ps.append(pool(**dict(dict(state=A + 0x10000000 * (l + 1)), **o.get("pool", {}))))
        Rs.append(records(**dict(dict(base=A + 0x10000000 * (l + 1) + 0x8000000), **o.get("rec", {}))))
    return ((_lib.KdaLayer * n)(*Ls), (_lib.KdaPool * n)(*Ps), (_lib.KdaRecords * n)(*Rs), n)


def commit_layers(arrs=None, n_rows=2, pending=None, eager=None, acc=A + 0x600000, cu=A, align=None):
    Ls, Ps, Rs, n = arrs or layer_arrays()
    al = None if align is None else ctypes.byref(align)
    return _lib.load().kda_commit_layers(Ls, Ps, Rs, n, cu, n_rows, None, acc, pending, eager, al, None)


def flush_layers(arrs=None, n_rows=2, pending=A + 0x700000):
    Ls, Ps, Rs, n = arrs or layer_arrays()
    return _lib.load().kda_flush_layers(Ls, Ps, Rs, n, n_rows, None, pending, None)


def test_commit_layers_validation():
    lib = _lib.load()
    Ls, Ps, Rs, n = layer_arrays()
    assert lib.kda_commit_layers(None, Ps, Rs, n, A, 2, None, A, None, None, None, None) == E["KDA_ERR_NULL"]
    assert commit_layers(layer_arrays(1), cu=0) == E["KDA_ERR_NULL"]
    assert commit_layers(layer_arrays(1), acc=0) == E["KDA_ERR_NULL"]
    assert lib.kda_commit_layers(Ls, Ps, Rs, 0, A, 2, None, A, None, None, None, None) == E["KDA_ERR_SHAPE"]
    assert commit_layers(layer_arrays(17)) == E["KDA_ERR_SHAPE"]
    assert commit_layers(layer_arrays(3, {1: {"layer": dict(num_heads=H + 1)}})) == E["KDA_ERR_SHAPE"]
    assert commit_layers(layer_arrays(3, {2: {"rec": dict(window=8)}})) == E["KDA_ERR_SHAPE"]
    assert commit_layers(layer_arrays(3, {1: {"pool": dict(state_indices=A + 0x500100)}})) == E["KDA_ERR_SHAPE"]
    assert commit_layers(layer_arrays(2, {1: {"layer": dict(head_dim=64)}})) == E["KDA_ERR_UNSUPPORTED"]
    assert commit_layers(eager=A + 0x700000) == E["KDA_ERR_SHAPE"]       # eager without pending
    assert commit_layers(n_rows=5) == E["KDA_ERR_CAPACITY"]
    assert commit_layers(n_rows=0) == E["KDA_OK"]                         # no rows: no launch


def test_commit_layers_aliasing():
    # two layers sharing one pool
    assert commit_layers(layer_arrays(2, {1: {"pool": dict(state=A + 0x10000000)}})) == E["KDA_ERR_ALIAS"]
    # a layer's records inside another layer's pool
    assert commit_layers(layer_arrays(2, {1: {"rec": dict(base=A + 0x10000000 + 0x1000)}})) == E["KDA_ERR_ALIAS"]
    # two layers' records overlapping
    assert commit_layers(layer_arrays(2, {1: {"rec": dict(base=A + 0x10000000 + 0x8000000 + 64)}})) == E["KDA_ERR_ALIAS"]
    # pending inside a pool
    assert commit_layers(pending=A + 0x20000000) == E["KDA_ERR_ALIAS"]


def test_flush_layers_validation():
    assert flush_layers(pending=0) == E["KDA_ERR_NULL"]
    assert flush_layers(layer_arrays(17)) == E["KDA_ERR_SHAPE"]
    assert flush_layers(layer_arrays(3, {1: {"rec": dict(rows=3)}})) == E["KDA_ERR_SHAPE"]
    assert flush_layers(pending=A + 0x30000000) == E["KDA_ERR_ALIAS"]    # pending inside a pool
    assert flush_layers(n_rows=5) == E["KDA_ERR_CAPACITY"]
    assert flush_layers(n_rows=0) == E["KDA_OK"]


def align(**kw):
    d = dict(block_table=A + 0x900000, row_stride=4, width=4, num_computed=A + 0x910000, block_size=16)
    d.update(kw)
    return _lib.KdaAlign(**d)


def test_commit_layers_align_validation():
    assert commit_layers(align=align(block_table=0)) == E["KDA_ERR_NULL"]
    assert commit_layers(align=align(num_computed=0)) == E["KDA_ERR_NULL"]
    assert commit_layers(align=align(width=0)) == E["KDA_ERR_SHAPE"]
    assert commit_layers(align=align(block_size=0)) == E["KDA_ERR_SHAPE"]
    assert commit_layers(align=align(row_stride=3)) == E["KDA_ERR_SHAPE"]
    # the deferred mode in align form passes the host checks (no rows: no launch)
    assert commit_layers(align=align(), pending=A + 0x700000, n_rows=0) == E["KDA_OK"]
    assert commit_layers(align=align(), n_rows=0) == E["KDA_OK"]


def conv_arrays(n=2, over=None):
    out = []
    for l in range(n):
        d = dict(state=A + 0x40000000 + l * 0x1000000, block_stride=3 * 6, dim_stride=6,
                 token_stride=1, num_blocks=8)
        d.update((over or {}).get(l, {}))
        out.append(_lib.KdaConvState(**d))
    return (_lib.KdaConvState * n)(*out), n


def conv(arrs=None, conv_dim=3, history=3, width=6, n_rows=2, window=4, al=None, cu=A,
         slots=A + 0x500000, acc=A + 0x600000):
    cs, n = arrs or conv_arrays()
    return _lib.load().kda_conv_compact(cs, n, conv_dim, history, width, cu, n_rows, slots, acc,
                                        window, None if al is None else ctypes.byref(al), None)


def test_conv_compact_validation():
    lib = _lib.load()
    assert lib.kda_conv_compact(None, 1, 3, 3, 6, A, 2, A, A, 4, None, None) == E["KDA_ERR_NULL"]
    assert conv(conv_arrays(1, {0: dict(state=0)})) == E["KDA_ERR_NULL"]
    assert conv(cu=0) == E["KDA_ERR_NULL"]
    assert conv(slots=0) == E["KDA_ERR_NULL"]
    assert conv(history=0) == E["KDA_ERR_SHAPE"]
    assert conv(history=9, width=16) == E["KDA_ERR_SHAPE"]
    assert conv(width=5) == E["KDA_ERR_SHAPE"]                 # < window + history - 1
    assert conv(window=0) == E["KDA_ERR_SHAPE"]
    assert conv(conv_dim=0) == E["KDA_ERR_SHAPE"]
    assert conv(conv_arrays(65)) == E["KDA_ERR_SHAPE"]
    assert conv(conv_arrays(1, {0: dict(token_stride=0)})) == E["KDA_ERR_SHAPE"]
    assert conv(conv_arrays(1, {0: dict(num_blocks=0)})) == E["KDA_ERR_SHAPE"]
    assert conv(conv_arrays(1, {0: dict(state=A + 0x40000001)})) == E["KDA_ERR_ALIGN"]
    assert conv(conv_arrays(2, {1: dict(state=A + 0x40000000 + 64)})) == E["KDA_ERR_ALIAS"]
    assert conv(al=align(width=0)) == E["KDA_ERR_SHAPE"]
    assert conv(n_rows=70000) == E["KDA_ERR_SHAPE"]
    assert conv(n_rows=0) == E["KDA_OK"]


def test_struct_layouts_match_the_header(tmp_path):
    """Every host struct of include/kda.h has the size and field offsets the
    ctypes binding assumes (compiled with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"kda_layer": _lib.KdaLayer, "kda_tokens": _lib.KdaTokens, "kda_pool": _lib.KdaPool,
               "kda_records": _lib.KdaRecords, "kda_align": _lib.KdaAlign,
               "kda_conv_state": _lib.KdaConvState, "kda_spec_table": _lib.KdaSpecTable}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "kda.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([cc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                          "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                         capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip(f"the header does not compile on the host here: {res.stderr[:200]}")
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, fname, val = line.split()
        got[(cname, fname)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, f"{cname}.{fname}"


# -------------------------------------------------- host metadata check --

def check_rows_c(cu, si, num_slots, num_tokens=None, rr=None, rec_rows=-1, max_seqlen=0):
    """kda_check_rows on host numpy arrays: (status, bad row, issue)."""
    import numpy as np
    lib = _lib.load()
    cu = np.ascontiguousarray(cu, np.int32)
    si = np.ascontiguousarray(si, np.int32)
    rr = None if rr is None else np.ascontiguousarray(rr, np.int32)
    bad, what = ctypes.c_int32(-7), ctypes.c_int32(-7)
    st = lib.kda_check_rows(cu.ctypes.data, len(cu) - 1, int(cu[-1]) if num_tokens is None else num_tokens,
                            si.ctypes.data, num_slots, None if rr is None else rr.ctypes.data,
                            rec_rows, max_seqlen, ctypes.byref(bad), ctypes.byref(what))
    return st, bad.value, what.value


def test_check_rows_accepts_good_metadata():
    # skipped rows (slot 0 and -1) may have any span and repeat slots
    cu = [0, 4, 8, 8, 11, 15]
    si = [3, 1, 0, -1, 2]
    assert check_rows_c(cu, si, 4, rr=[2, -1, 0, 0, 1], rec_rows=3, max_seqlen=4) == (0, -1, 0)
    assert check_rows_c(cu, si, 4) == (0, -1, 0)                      # no record check
    assert check_rows_c([0], [], 4)[0] == 0                           # no rows


def test_check_rows_names_the_first_bad_row():
    M = E["KDA_ERR_METADATA"]
    # spans
    assert check_rows_c([0, 4, 3, 8], [1, 2, 3], 4) == (M, 1, 1)      # end before start
    assert check_rows_c([0, 4, 8, 12], [1, 2, 3], 4, num_tokens=10) == (M, 2, 1)   # beyond the tokens
    assert check_rows_c([-1, 4, 8], [1, 2], 4) == (M, 0, 1)           # negative start
    # window longer than the bound
    assert check_rows_c([0, 4, 9, 12], [1, 2, 3], 4, max_seqlen=4) == (M, 1, 2)
    # slots
    assert check_rows_c([0, 1, 2, 3], [1, 4, 2], 4) == (M, 1, 3)      # slot >= num_slots
    assert check_rows_c([0, 1, 2, 3], [1, 2, 1], 4) == (M, 2, 4)      # shared slot
    # record rows
    assert check_rows_c([0, 1, 2, 3], [1, 2, 3], 4, rr=[0, 3, 1], rec_rows=3) == (M, 1, 5)
    assert check_rows_c([0, 1, 2, 3], [1, 2, 3], 4, rr=[0, -2, 1], rec_rows=3) == (M, 1, 5)
    assert check_rows_c([0, 1, 2, 3], [1, 2, 3], 4, rr=[0, 1, 0], rec_rows=3) == (M, 2, 6)
    assert check_rows_c([0, 1, 2, 3], [1, 2, 3], 4, rr=[-1, -1, 1], rec_rows=3) == (0, -1, 0)
    # identity record rows beyond the record rows
    assert check_rows_c([0, 1, 2, 3], [1, 2, 3], 4, rec_rows=2) == (M, 2, 5)


def test_check_rows_argument_errors():
    lib = _lib.load()
    import numpy as np
    cu = np.zeros(3, np.int32)
    assert lib.kda_check_rows(None, 2, 0, cu.ctypes.data, 4, None, -1, 0, None, None) == E["KDA_ERR_NULL"]
    assert lib.kda_check_rows(cu.ctypes.data, -1, 0, cu.ctypes.data, 4, None, -1, 0, None, None) == E["KDA_ERR_SHAPE"]
    assert lib.kda_check_rows(cu.ctypes.data, 2, 0, cu.ctypes.data, 4, None, -1, -3, None, None) == E["KDA_ERR_SHAPE"]


def test_binding_check_rows_raises_with_the_row():
    import torch
    import linear_attention_speculative_kda_amd as kda
    cu = torch.tensor([0, 4, 8, 12], dtype=torch.int32)
    kda.check_rows(cu, torch.tensor([1, 2, 3], dtype=torch.int32), num_slots=4, max_seqlen=4)
    with pytest.raises(_lib.KdaError, match="row 2: slot shared"):
        kda.check_rows(cu, torch.tensor([1, 2, 1], dtype=torch.int32), num_slots=4)
    with pytest.raises(_lib.KdaError, match="row 0: window longer"):
        kda.check_rows(cu, torch.tensor([1, 2, 3], dtype=torch.int32), num_slots=4, max_seqlen=3)
