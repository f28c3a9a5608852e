"""The accuracy study's pieces (oracle/accuracy.py) against closed forms and the pages.

CPU only.  Pins: Eq. 4 on exactly representable groups, its error bound and the
effective-bins count of Eq. 5 (technical review 'Lynx: Progressive Speculative KV
Cache Transfer for Disaggregated LLM Inference', Prerequisites §4); the bit-split
generalisation of Stage 4 by exhaustion; the vNMSE definition on hand cases; the
qualitative ordering of the pages' vNMSE table; and the stored table
(tests/golden/accuracy_vnmse.txt, written by tests/golden/make_accuracy_table.py).
"""
import os

import numpy as np
import pytest

from decode_attention_lynx_amd import synth
from oracle import accuracy as acc
from oracle import lynx_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accuracy_vnmse.txt")


def test_linear_exact_on_its_grid():
    x = (np.arange(16) * 0.5 + 3.0)[None, :]
    Q, S, Z = acc.linear_codes(x, 4)
    assert S.item() == 0.5 and Z.item() == -6.0
    assert np.array_equal(Q[0], np.arange(16))
    assert np.array_equal(acc.linear_roundtrip(x, 4), x)
    c = np.full((1, 8), -2.5)                               # constant group: exact
    assert np.array_equal(acc.linear_roundtrip(c, 8), c)


@pytest.mark.parametrize("bits", [4, 8])
def test_linear_error_bound(bits):
    rng = np.random.default_rng(bits)
    x = rng.laplace(0.0, 1.0, size=(500, 128)) + rng.normal(0, 3, size=(500, 1))
    Q, S, Z = acc.linear_codes(x, bits)
    assert Q.min() >= 0 and Q.max() <= 2 ** bits - 1
    err = np.abs(acc.linear_roundtrip(x, bits) - x)
    # rounding costs at most S/2; the rounded zero point can push an extreme value by S/2 more
    assert np.all(err <= S * (1.0 + 1e-12))
    inner = (x > x.min(-1, keepdims=True) + S) & (x < x.max(-1, keepdims=True) - S)
    assert np.all(err[inner] <= (S * 0.5 * (1 + 1e-12) * np.ones_like(x))[inner])


def test_effective_bins_of_eq5():
    """Outlier channels 100x the others (the token spans [-100, 100]): the ordinary channels,
    in [-1, 1], of an INT8 token fall in about 2^B m_i / m = 2.56 of the 256 levels (Eq. 5)."""
    rng = np.random.default_rng(5)
    x = rng.uniform(-1.0, 1.0, size=(200, 128))
    x[:, 7], x[:, 9] = 100.0, -100.0
    Q, _, _ = acc.linear_codes(x, 8)
    used = [len(np.unique(np.delete(Q[t], [7, 9]))) for t in range(200)]
    assert 2.5 <= np.mean(used) <= 3.6


def test_split_anchor_code_by_exhaustion():
    I = np.arange(128)
    for a in (3, 4, 5, 6, 7):
        Ia = acc.split_anchor_code(I, a)
        res = Ia - I
        r = 8 - a
        assert res.min() == -(2 ** (r - 1)) and res.max() == 2 ** (r - 1) - 1   # fits r signed bits
        assert np.array_equal(Ia >> r, I >> r)                                   # the anchor keeps the top bits
    assert np.array_equal(acc.split_anchor_code(I, 8), I)
    # a = 4 is the codec's own anchor-only code, 16 V_mag + 7 (reading R-split)
    S = np.ones(128, dtype=np.int32)
    Q_anc, _ = o.split_streams(I, S)
    assert np.array_equal(acc.split_anchor_code(I, 4), o.code_anchor_only(Q_anc)[1])


def test_int8_split_anchor_bound():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1, size=(300, 128))
    _, S, _ = acc.linear_codes(x, 8)
    assert np.all(np.abs(acc.int8_split_anchor(x) - x) <= 8.0 * S * (1 + 1e-12))


def test_vnmse_definition():
    O = np.array([[1.0, 0.0], [0.0, 1.0]])
    assert acc.vnmse(O, O) == 0.0
    assert acc.vnmse(np.array([[1.0, 1.0], [0.0, 1.0]]), O) == 0.5
    rng = np.random.default_rng(1)
    A, B = rng.normal(size=(3, 5)), rng.normal(size=(3, 5))
    assert abs(acc.vnmse(3.0 * A, 3.0 * B) - acc.vnmse(A, B)) < 1e-15


def small_inputs(scale):
    T, Hkv, Hq, M = 1024, 2, 16, 4
    k = synth.make_kv_np(T, Hkv, 128, seed=11, layer=0, kv_idx=0)
    v = synth.make_kv_np(T, Hkv, 128, seed=11, layer=0, kv_idx=1)
    q = o.f64_to_bf16_bits(o.bf16_bits_to_f64(synth.make_q_np(M, Hq, 128, seed=11)) * scale).reshape(1, M, Hq, 128)
    return k, v, q, T


def test_study_ordering_soft_softmax():
    """With a soft softmax (query scale 0.03) the ordering is the pages' one:
    Lynx < INT8 < Lynx-INT4 < INT4; more anchor bits never hurt the draft."""
    k, v, q, T = small_inputs(0.03)
    r = acc.study(k, v, q, T, 256, 64, 255.0)
    assert r["Lynx"] < r["INT8"] < r["Lynx-INT4"] < r["INT4"]
    assert r["Lynx anchor 6+2"] < r["Lynx anchor 5+3"] < r["Lynx-INT4"] < r["Lynx anchor 3+5"]


def test_study_ordering_sharp_softmax():
    """With N(0,1) queries (logit std ~13 on this KV) the full stream still beats INT8 and INT4,
    but the 3-bit-magnitude anchor loses to per-token INT4, whose scale is set by the outlier
    channels that dominate such scores."""
    k, v, q, T = small_inputs(1.0)
    r = acc.study(k, v, q, T, 256, 64, 255.0)
    assert r["Lynx"] < r["INT8"] < r["INT4"] < r["Lynx-INT4"]
    assert r["Lynx anchor 6+2"] < r["Lynx anchor 5+3"] < r["Lynx-INT4"] < r["Lynx anchor 3+5"]


def read_golden():
    methods, section = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            section = line
            continue
        if section == "[methods]" and not line.startswith("method"):
            name, *vals = [x.strip() for x in line.split("|")]
            methods[name] = [float(x) for x in vals]
    return methods


def test_golden_table_reproduces():
    """Recompute the query-scale-0.03 column of the stored table."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("mk", os.path.join(os.path.dirname(GOLDEN),
                                                                     "make_accuracy_table.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    k, v, q = mk.inputs()
    col = mk.Q_SCALES.index(0.03)
    r = acc.study(k, v, mk.scaled(q, 0.03), mk.T, 256, 64, 255.0)
    stored = read_golden()
    assert set(stored) == set(r)
    for name, vals in stored.items():
        assert abs(vals[col] - r[name]) <= 1e-4 * r[name], name
