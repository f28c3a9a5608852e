"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

from decode_attention_lynx_amd import lynx
from oracle import lynx_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lynx.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(lynx_\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_exports_declared_symbols():
    L = lynx.lib()
    syms = declared_symbols()
    assert set(syms) == set(lynx.EXPORTS), syms
    for s in syms:
        assert hasattr(L, s), s


def test_strerror():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lynx.strerror(st), str) and lynx.strerror(st)


@pytest.mark.parametrize("P,Hkv,D,C", [(256, 8, 128, 64), (4096, 8, 128, 64), (256, 4, 128, 32),
                                       (256, 1, 128, 256), (24, 3, 128, 8), (256, 128, 1, 32)])
def test_stream_sizes_match_oracle(P, Hkv, D, C):
    assert lynx.stream_sizes(P, Hkv, D, C) == o.segment_bytes(P, Hkv, D, C)


def test_stream_sizes_rejects():
    for args in [(0, 8, 128, 64), (256, 8, 128, 48), (256, 0, 128, 64), (256, 8, 128, 0), (3, 1, 1, 1)]:
        with pytest.raises(lynx.LynxError):
            lynx.stream_sizes(*args)


# --------------------------------------------------------------------------
# argument validation: every case returns before any HIP call
# --------------------------------------------------------------------------
GOOD = ctypes.c_void_p(0x10000)        # an aligned dummy address; never dereferenced on error paths
ODD = ctypes.c_void_p(0x10008)


def enc(n_pages=1, P=256, Hkv=8, D=128, C=64, alpha=255.0, sel=3, kv=GOOD, anc=GOOD, res=GOOD):
    return lynx.lib().lynx_encode(kv, n_pages, P, Hkv, D, C, alpha, sel, anc, res, None)


def test_encode_validation():
    assert enc(n_pages=-1) == lynx.LYNX_EINVAL
    assert enc(P=0) == lynx.LYNX_EINVAL
    assert enc(Hkv=0) == lynx.LYNX_EINVAL
    assert enc(P=96, C=64) == lynx.LYNX_EINVAL                 # P % C
    for a in (0.0, -1.0, float("nan"), float("inf")):
        assert enc(alpha=a) == lynx.LYNX_EINVAL
    assert enc(sel=0) == lynx.LYNX_EINVAL
    assert enc(sel=2) == lynx.LYNX_EINVAL                      # anchor (metadata) is required
    assert enc(sel=5) == lynx.LYNX_EINVAL
    assert enc(D=64) == lynx.LYNX_EUNSUPPORTED
    assert enc(P=96, C=48) == lynx.LYNX_EUNSUPPORTED           # chunk not a power of two in [8, 256]
    assert enc(P=1024, C=512) == lynx.LYNX_EUNSUPPORTED
    assert enc(P=4, C=4) == lynx.LYNX_EUNSUPPORTED
    assert enc(kv=None) == lynx.LYNX_EALIGN
    assert enc(anc=ODD) == lynx.LYNX_EALIGN
    assert enc(res=None) == lynx.LYNX_EALIGN                   # residual selected but missing
    assert enc(n_pages=0, kv=None, anc=None, res=None) == lynx.LYNX_OK   # empty input: no-op


def test_decode_validation():
    L = lynx.lib()
    da = lambda **k: L.lynx_decode_anchor(k.get("anc", GOOD), k.get("n", 1), k.get("P", 256), 8, k.get("D", 128),
                                          k.get("C", 64), k.get("alpha", 255.0), k.get("dt", 0), k.get("out", GOOD),
                                          None)
    df = lambda **k: L.lynx_decode_full(k.get("anc", GOOD), k.get("res", GOOD), k.get("n", 1), 256, 8, 128, 64,
                                        255.0, k.get("dt", 1), k.get("out", GOOD), None)
    assert da(dt=2) == lynx.LYNX_EINVAL
    assert da(n=-3) == lynx.LYNX_EINVAL
    assert da(alpha=float("nan")) == lynx.LYNX_EINVAL
    assert da(P=100, C=64) == lynx.LYNX_EINVAL
    assert da(D=256) == lynx.LYNX_EUNSUPPORTED
    assert da(out=ODD) == lynx.LYNX_EALIGN
    assert da(anc=None) == lynx.LYNX_EALIGN
    assert da(n=0, anc=None, out=None) == lynx.LYNX_OK
    assert df(res=None) == lynx.LYNX_EALIGN
    assert df(dt=-1) == lynx.LYNX_EINVAL
    assert df(n=0, anc=None, res=None, out=None) == lynx.LYNX_OK
