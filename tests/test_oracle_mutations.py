"""The pins are sharp: each planted mistake in a copy of the oracle fails one.

A copy of ``oracle/gdn2_oracle.c`` is edited on the CPU (a flipped sign, a
dropped decay, the read taken before the decay, the output read before the
update, the erase gate moved off the key axis) and compiled into a temporary
library; the worked examples and closed forms that pin the real oracle must
then reject it.  The real oracle is never modified.
"""
import ctypes
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn2_oracle.c")

DECAY_BLOCK = """            /* 1. decay each key row of the state */
            for (int64_t i = 0; i < dk; ++i) {
                const double la = decay_per_key ? log_decay[row * dk + i] : log_decay[row];
                const double a = exp(la);
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
            }
"""
READ_BLOCK = """            /* 2. read the decayed state along the key: m = Sbar^T k */
            for (int64_t j = 0; j < dv; ++j) m[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) m[j] += S[i * dv + j] * kt[i];
"""
OUT_START = "            /* 4. read the updated state with the query */"
ERASE_START = "            /* 3. erase (b .* k) m^T, write (w .* k) v^T */"
OUT_BLOCK = """            /* 4. read the updated state with the query */
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double qi = q_scale * qt[i];
                for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qi;
            }
"""

MUTANTS = {
    "erase_sign_flipped": [("S[i * dv + j] - ei * m[j]", "S[i * dv + j] + ei * m[j]")],
    "no_decay": [("const double a = exp(la);", "const double a = 1.0 + 0.0 * la;")],
    "read_before_decay": [(DECAY_BLOCK + READ_BLOCK, READ_BLOCK + DECAY_BLOCK)],
    "write_not_gated": [("const double ui = wi * kt[i];", "const double ui = kt[i];")],
    "erase_gate_on_value_axis": [
        ("const double ei = bi * kt[i];", "const double ei = kt[i];"),
        ("S[i * dv + j] - ei * m[j]", "S[i * dv + j] - ei * m[j] * (erase_per_key ? erase[row * dk + (j % dk)] : bi)"),
    ],
    "output_read_before_update": [(OUT_BLOCK, ""), (ERASE_START, OUT_BLOCK + ERASE_START)],
    "decay_after_write": [(DECAY_BLOCK + READ_BLOCK, READ_BLOCK),
                          (OUT_START, DECAY_BLOCK + OUT_START)],
    # the value-write form (gist.science summary's equation)
    "value_write_read_not_gated": [("m[j] += S[i * dv + j] * bi * kt[i];", "m[j] += S[i * dv + j] * kt[i];")],
    "value_write_gate_on_key": [("const double wj = write_per_key ? write[row * dv + j] : write[row];",
                                 "const double wj = write_per_key ? write[row * dv + (i % dv)] : write[row];")],
}


def _build(tmp, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert old in text, f"mutation anchor missing for {name}"
        text = text.replace(old, new, 1)
    src = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    open(src, "w").write(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", src, "-o", lib, "-lm"], check=True)
    L = ctypes.CDLL(lib)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    L.gdn2_oracle_fwd.restype = ctypes.c_int
    L.gdn2_oracle_fwd.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp, ctypes.c_int,
                                  dp, ctypes.c_int, dp, ctypes.c_int, dp, ctypes.c_double,
                                  dp, dp, ctypes.c_int, ctypes.c_int]
    return L


def _run(L, q, k, v, la, b, w, S0, form=0):
    arrs = [np.ascontiguousarray(x, dtype=np.float64) if x is not None else None
            for x in (q, k, v, la, b, w, S0)]
    q, k, v, la, b, w, S0 = arrs
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    p = lambda x: None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    kind = lambda g: 1 if g.ndim == 4 else 0
    rc = L.gdn2_oracle_fwd(B, T, H, dk, dv, p(q), p(k), p(v), p(la), kind(la), p(b), kind(b),
                           p(w), 0 if w is None else kind(w), p(S0), 1.0, p(o), p(S), form, 1)
    assert rc == 0
    return o, S


def _pins_pass(L):
    """The page pins and two closed forms, as booleans."""
    ok = []
    # scalar example: 4 -> 4 with alpha .5, beta .25, value 10
    o, S = _run(L, [[[[1.0]]]], [[[[1.0]]]], [[[[10.0]]]], np.full((1, 1, 1), math.log(0.5)),
                np.full((1, 1, 1), 0.25), None, [[[[4.0]]]])
    ok.append(abs(S[0, 0, 0, 0] - 4.0) < 1e-9 and abs(o[0, 0, 0, 0] - 4.0) < 1e-9)
    # 2x2 trace
    o, S = _run(L, np.array([1.0, 0]).reshape(1, 1, 1, 2), np.array([1.0, 0]).reshape(1, 1, 1, 2),
                np.array([9.0, 9]).reshape(1, 1, 1, 2), np.full((1, 1, 1), math.log(0.8)),
                np.full((1, 1, 1), 0.5), None, np.array([[2.0, 3], [5, 1]]).reshape(1, 1, 2, 2))
    ok.append(np.allclose(S[0, 0], [[5.3, 5.7], [4.0, 0.8]], atol=1e-9)
              and np.allclose(o[0, 0, 0], [5.3, 5.7], atol=1e-9))
    # one-hot key with per-channel erase/write gates, dk != dv
    r = np.random.Generator(np.random.PCG64(5))
    dk, dv = 3, 5
    S0 = r.normal(size=(1, 1, dk, dv))
    k = np.zeros((1, 1, 1, dk)); k[..., 1] = 1.0
    la = -r.uniform(0, 1, size=(1, 1, 1, dk))
    b = r.uniform(size=(1, 1, 1, dk)); w = r.uniform(size=(1, 1, 1, dk))
    v = r.normal(size=(1, 1, 1, dv)); q = r.normal(size=(1, 1, 1, dk))
    o, S = _run(L, q, k, v, la, b, w, S0)
    a = np.exp(la[0, 0, 0])
    ref = a[:, None] * S0[0, 0]
    ref[1] = a[1] * (1 - b[0, 0, 0, 1]) * S0[0, 0, 1] + w[0, 0, 0, 1] * v[0, 0, 0]
    ok.append(np.allclose(S[0, 0], ref, atol=1e-12))
    # full erase with unit keys reads back sum_c w_c k_c^2 times v
    T = 4
    kk = r.normal(size=(1, T, 1, dk)); kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    la = -r.uniform(0, 1, size=(1, T, 1, dk)); w = r.uniform(size=(1, T, 1, dk))
    v = r.normal(size=(1, T, 1, dv))
    o, S = _run(L, kk, kk, v, la, np.ones((1, T, 1, dk)), w, r.normal(size=(1, 1, dk, dv)))
    gain = np.sum(w * kk ** 2, axis=-1)
    ok.append(np.allclose(o, gain[..., None] * v, atol=1e-11))
    # the value-write form, worked by hand (tests/test_oracle_value_write.py)
    o, S = _run(L, np.array([1.0, 0]).reshape(1, 1, 1, 2), np.array([0.6, 0.8]).reshape(1, 1, 1, 2),
                np.array([9.0, 9]).reshape(1, 1, 1, 2), np.full((1, 1, 1), math.log(0.8)),
                np.array([0.5, 1.0]).reshape(1, 1, 1, 2), np.array([1.0, 0.5]).reshape(1, 1, 1, 2),
                np.array([[2.0, 3], [5, 1]]).reshape(1, 1, 2, 2), form=1)
    ok.append(np.allclose(S[0, 0], [[4.792, 4.284], [8.256, 3.312]], atol=1e-12))
    return all(ok)


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="gdn2_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes(tmpdir_mod):
    assert _pins_pass(_build(tmpdir_mod, "original", []))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmpdir_mod, name):
    assert not _pins_pass(_build(tmpdir_mod, name, MUTANTS[name]))
