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


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built library every entry point raises instead of computing."""
    monkeypatch.setattr(lynx, "_lib", None)
    monkeypatch.setattr(lynx, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "liblynx.so"))
    with pytest.raises(RuntimeError, match="not found"):
        lynx.lib()
    with pytest.raises(RuntimeError, match="not found"):
        lynx.stream_sizes(256, 8, 128, 64)
    with pytest.raises(RuntimeError, match="not found"):
        lynx.attn_workspace_bytes(16, 32768, 64, 8, 128, 256, 64)


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
    # encoder workgroups beyond int: (page, head, slab, 256-token tile) units of long pages
    # (8388608 pages x 80 heads x 2 slabs x 2 tiles; the decoders' 3 tiles of 128 still fit)
    assert enc(n_pages=1 << 23, P=264, Hkv=80, C=8) == lynx.LYNX_EUNSUPPORTED
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


def attn(B=2, T=1024, Hq=16, Hkv=2, D=128, P=256, C=64, alpha=255.0, sm=0.0, ws_bytes=None, dt=lynx.OUT_F32,
         q=GOOD, k=GOOD, v=GOOD, ws=GOOD, out=GOOD):
    if ws_bytes is None:
        ws_bytes = 0       # too small for any supported case: the ENOSPACE check comes before any launch
    return lynx.lib().lynx_attn_anchor(q, k, v, B, T, Hq, Hkv, D, P, C, alpha, sm, ws, ws_bytes, dt, out, None)


def test_attention_validation():
    assert attn(T=1000) == lynx.LYNX_EINVAL                    # ctx % P
    assert attn(P=96, C=64) == lynx.LYNX_EINVAL                # P % C
    assert attn(Hq=15) == lynx.LYNX_EINVAL                     # Hq % Hkv
    assert attn(alpha=0.0) == lynx.LYNX_EINVAL
    assert attn(alpha=float("nan")) == lynx.LYNX_EINVAL
    assert attn(sm=float("inf")) == lynx.LYNX_EINVAL
    assert attn(dt=5) == lynx.LYNX_EINVAL
    assert attn(T=0) == lynx.LYNX_EINVAL
    assert attn(D=64) == lynx.LYNX_EUNSUPPORTED
    assert attn(C=16, P=256) == lynx.LYNX_ENOSPACE              # chunk 16: supported, workspace too small
    assert attn(C=16, P=96, T=960) == lynx.LYNX_EUNSUPPORTED    # chunk 16 in pages of no whole 64-token tile
    assert attn(C=8, P=256) == lynx.LYNX_ENOSPACE               # chunk 8: supported
    assert attn(C=8, P=48, T=960) == lynx.LYNX_EUNSUPPORTED     # chunk 8 in pages of no whole 32-token tile
    assert attn(Hq=32, Hkv=2) == lynx.LYNX_ENOSPACE             # group of 16: supported
    assert attn(Hq=34, Hkv=2) == lynx.LYNX_EUNSUPPORTED         # group of 17 query heads
    assert attn(q=ODD) == lynx.LYNX_EALIGN
    assert attn(out=None) == lynx.LYNX_EALIGN
    assert attn(ws=ODD) == lynx.LYNX_EALIGN
    assert attn() == lynx.LYNX_ENOSPACE
    assert attn(C=32) == lynx.LYNX_ENOSPACE                     # chunk 32: supported, workspace too small
    assert attn(B=0) == lynx.LYNX_OK                            # nothing to do


@pytest.mark.parametrize("B,T,Hq,Hkv,P,C", [(16, 32768, 64, 8, 256, 64), (2, 1024, 16, 2, 256, 64),
                                            (3, 320, 8, 1, 64, 64), (2, 512, 8, 2, 256, 32), (1, 64, 2, 2, 64, 64),
                                            (1, 96, 8, 1, 32, 32), (2, 512, 32, 2, 256, 16), (1, 96, 8, 1, 32, 8)])
def test_attention_workspace_bytes(B, T, Hq, Hkv, P, C):
    """One (m, l, o[128]) float32 record per (sequence, query head, context split); the splits
    cover the context's tiles with no empty split."""
    ws = lynx.attn_workspace_bytes(B, T, Hq, Hkv, 128, P, C)
    rec = (128 + 2) * 4
    assert ws > 0 and ws % (B * Hq * rec) == 0
    splits = ws // (B * Hq * rec)
    tile = 64 if C % 64 == 0 or (C in (16, 32) and P % 64 == 0) else 32
    ntiles = T // tile
    per = -(-ntiles // splits)
    assert 1 <= splits <= ntiles and (splits - 1) * per < ntiles <= splits * per


def test_attention_workspace_bytes_unsupported():
    assert lynx.attn_workspace_bytes(2, 960, 16, 2, 128, 96, 16) == 0
    assert lynx.attn_workspace_bytes(2, 1024, 34, 2, 128, 256, 64) == 0
    assert lynx.attn_workspace_bytes(2, 1000, 16, 2, 128, 256, 64) == 0
    assert lynx.attn_workspace_bytes(2, 1024, 16, 2, 64, 256, 64) == 0


def verify(B=2, M=4, T=1024, Hq=16, Hkv=2, D=128, P=256, C=64, alpha=255.0, sm=0.0, dt=lynx.OUT_F32, q=GOOD,
           k=GOOD, kr=GOOD, v=GOOD, vr=GOOD, ws=GOOD, out=GOOD, lse=None):
    # workspace size 0: too small for any supported case, so no call below reaches a launch
    return lynx.lib().lynx_attn_verify(q, k, kr, v, vr, B, M, T, Hq, Hkv, D, P, C, alpha, sm, ws, 0, dt, out, lse,
                                       None)


def test_verify_validation():
    assert verify(T=1000) == lynx.LYNX_EINVAL                  # ctx % P
    assert verify(P=96, C=64) == lynx.LYNX_EINVAL              # P % C
    assert verify(Hq=15) == lynx.LYNX_EINVAL                   # Hq % Hkv
    assert verify(M=0) == lynx.LYNX_EINVAL
    assert verify(alpha=-1.0) == lynx.LYNX_EINVAL
    assert verify(sm=float("nan")) == lynx.LYNX_EINVAL
    assert verify(dt=3) == lynx.LYNX_EINVAL
    assert verify(D=64) == lynx.LYNX_EUNSUPPORTED
    assert verify(C=16, P=256) == lynx.LYNX_ENOSPACE            # chunk 16: supported
    assert verify(C=8, P=256) == lynx.LYNX_EUNSUPPORTED         # chunk 8: not in the verification kernel
    assert verify(T=960, P=96, C=32) == lynx.LYNX_EUNSUPPORTED   # chunk 32 in pages of 96: tiles cross pages
    assert verify(C=32, P=256) == lynx.LYNX_ENOSPACE             # chunk 32: supported
    assert verify(kr=ODD) == lynx.LYNX_EALIGN
    assert verify(vr=None) == lynx.LYNX_EALIGN
    assert verify(lse=ctypes.c_void_p(GOOD.value + 2)) == lynx.LYNX_EALIGN
    assert verify() == lynx.LYNX_ENOSPACE
    assert verify(lse=GOOD) == lynx.LYNX_ENOSPACE
    assert verify(B=0) == lynx.LYNX_OK                          # nothing to do


@pytest.mark.parametrize("B,M,T,Hq,Hkv,P,C", [(16, 64, 32768, 64, 8, 256, 64), (2, 4, 1024, 16, 2, 256, 64),
                                              (1, 17, 256, 64, 8, 256, 64), (3, 1, 320, 8, 1, 64, 64),
                                              (2, 5, 512, 12, 4, 256, 128), (2, 4, 1024, 16, 2, 256, 32),
                                              (2, 4, 1024, 64, 4, 256, 16)])
def test_verify_workspace_bytes(B, M, T, Hq, Hkv, P, C):
    """One (m, l, 0, 0, o[128]) float32 record per (sequence, draft token, query head, context split);
    the splits cover the context's 64-token tiles with no empty split."""
    ws = lynx.attn_verify_workspace_bytes(B, M, T, Hq, Hkv, 128, P, C)
    rec = (128 + 4) * 4
    assert ws > 0 and ws % (B * M * Hq * rec) == 0
    splits = ws // (B * M * Hq * rec)
    ntiles = T // 64
    per = -(-ntiles // splits)
    assert 1 <= splits <= ntiles and (splits - 1) * per < ntiles <= splits * per


def test_verify_workspace_bytes_unsupported():
    assert lynx.attn_verify_workspace_bytes(2, 4, 1024, 16, 2, 128, 256, 8) == 0
    assert lynx.attn_verify_workspace_bytes(2, 4, 960, 16, 2, 128, 96, 32) == 0
    assert lynx.attn_verify_workspace_bytes(2, 4, 1000, 16, 2, 128, 256, 64) == 0
    assert lynx.attn_verify_workspace_bytes(2, 0, 1024, 16, 2, 128, 256, 64) == 0
    assert lynx.attn_verify_workspace_bytes(2, 4, 1024, 16, 2, 64, 256, 64) == 0


def paged(B=2, maxp=4, Hq=16, Hkv=2, D=128, P=256, C=64, n_pool=8, alpha=255.0, bt=GOOD, sl=GOOD, q=GOOD,
          k=GOOD, v=GOOD, ws=GOOD, out=GOOD):
    # workspace size 0: too small for any supported case, so no call below reaches a launch
    return lynx.lib().lynx_attn_anchor_paged(q, k, v, n_pool, bt, sl, B, maxp, Hq, Hkv, D, P, C, alpha, 0.0, ws, 0,
                                             lynx.OUT_F32, out, None)


def test_attention_paged_validation():
    assert paged(n_pool=0) == lynx.LYNX_EINVAL
    assert paged(maxp=0) == lynx.LYNX_EINVAL
    assert paged(P=96, C=64) == lynx.LYNX_EINVAL                 # P % C
    assert paged(bt=None) == lynx.LYNX_EALIGN
    assert paged(sl=ctypes.c_void_p(GOOD.value + 2)) == lynx.LYNX_EALIGN
    assert paged(D=64) == lynx.LYNX_EUNSUPPORTED
    assert paged(maxp=1 << 24) == lynx.LYNX_EUNSUPPORTED          # max_pages * P overflows int
    assert paged() == lynx.LYNX_ENOSPACE
    assert paged(B=0) == lynx.LYNX_OK


def test_encode_to_host_validation_and_staging():
    L = lynx.lib()
    a, r = lynx.stream_sizes(256, 2, 128, 64)
    assert L.lynx_encode_to_host_staging_bytes(4, 256, 2, 128, 64) == 2 * 4 * (a + r)
    assert L.lynx_encode_to_host_staging_bytes(0, 256, 2, 128, 64) == 0
    assert L.lynx_encode_to_host_staging_bytes(4, 256, 2, 64, 64) == 0

    def call(n=4, gp=2, staging=GOOD, sbytes=1 << 40, ah=GOOD, rh=GOOD, C=64, kv=GOOD):
        return L.lynx_encode_to_host(kv, n, 256, 2, 128, C, 255.0, gp, staging, sbytes, ah, rh, None, None)
    assert call(gp=0) == lynx.LYNX_EINVAL
    assert call(ah=None) == lynx.LYNX_EINVAL
    assert call(C=48) == lynx.LYNX_EINVAL                    # P % C
    assert call(C=12) == lynx.LYNX_EINVAL                    # 256 % 12 != 0
    assert call(staging=ODD) == lynx.LYNX_EALIGN
    assert call(kv=ODD) == lynx.LYNX_EALIGN
    assert call(sbytes=2 * 2 * (a + r) - 1) == lynx.LYNX_ENOSPACE
    assert call(n=0) == lynx.LYNX_OK


def test_verify_paged_validation():
    def call(B=2, M=4, maxp=4, n_pool=8, bt=GOOD, sl=GOOD, P=256, C=64, D=128):
        return lynx.lib().lynx_attn_verify_paged(GOOD, GOOD, GOOD, GOOD, GOOD, n_pool, bt, sl, B, M, maxp, 16, 2, D,
                                                 P, C, 255.0, 0.0, GOOD, 0, lynx.OUT_F32, GOOD, None, None)
    assert call(n_pool=0) == lynx.LYNX_EINVAL
    assert call(maxp=0) == lynx.LYNX_EINVAL
    assert call(bt=None) == lynx.LYNX_EALIGN
    assert call(sl=ctypes.c_void_p(GOOD.value + 2)) == lynx.LYNX_EALIGN
    assert call(C=8) == lynx.LYNX_EUNSUPPORTED
    assert call(maxp=1 << 24) == lynx.LYNX_EUNSUPPORTED
    assert call() == lynx.LYNX_ENOSPACE
    assert call(B=0) == lynx.LYNX_OK


def test_geometry_too_large_for_int_sizes():
    """A page whose byte count does not fit an int is refused before any launch."""
    L = lynx.lib()
    assert L.lynx_encode(GOOD, 1, 1 << 16, 1 << 12, 128, 64, 255.0, 3, GOOD, GOOD, None) == lynx.LYNX_EUNSUPPORTED
    assert L.lynx_decode_full(GOOD, GOOD, 1, 1 << 16, 1 << 12, 128, 64, 255.0, lynx.OUT_BF16, GOOD, None) == \
        lynx.LYNX_EUNSUPPORTED


def test_binding_refuses_buffers_before_any_launch():
    """The binding checks device, dtype, contiguity and sizes of the tensors it passes as
    pointers; these cases raise on the host without touching a GPU."""
    import torch
    kv_host = torch.zeros((256, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        lynx.encode(kv_host, 256, 64, 255.0)
    with pytest.raises(ValueError, match="whole number"):
        lynx.encode(torch.zeros((300, 2, 128), dtype=torch.bfloat16), 256, 64, 255.0)
    a_sz, _ = lynx.stream_sizes(256, 2, 128, 64)
    with pytest.raises(ValueError, match="CUDA"):
        lynx.decode_anchor(torch.zeros((1, a_sz), dtype=torch.uint8), 1, 256, 2, 128, 64, 255.0)
    with pytest.raises(ValueError, match="dtype"):
        lynx._need(torch.zeros(4, dtype=torch.float16), "out", 0, (torch.bfloat16, torch.float32), device="cpu")
    with pytest.raises(ValueError, match="contiguous"):
        lynx._need(torch.zeros((4, 4)).t(), "x", 0, device="cpu")
    with pytest.raises(ValueError, match="bytes"):
        lynx._need(torch.zeros(4, dtype=torch.uint8), "x", 5, device="cpu")
    assert lynx._need(torch.zeros(5, dtype=torch.uint8), "x", 5, device="cpu") is not None


def test_attention_noalloc_validation():
    """The no-allocation entry point refuses, on the host and before any launch, a shape whose
    partial results exceed its per-GPU buffer, and reports argument errors as lynx_attn_anchor."""
    def call(B=2, T=1024, Hq=16, Hkv=2, P=256, C=64, dt=lynx.OUT_F32, q=GOOD, out=GOOD):
        return lynx.lib().lynx_attn_anchor_noalloc(q, GOOD, GOOD, B, T, Hq, Hkv, 128, P, C, 255.0, 0.0, dt, out,
                                                   None)
    assert lynx.attn_workspace_bytes(1024, 256, 64, 8, 128, 256, 64) > lynx.ATTN_SCRATCH_BYTES
    assert call(B=1024, T=256, Hq=64, Hkv=8) == lynx.LYNX_ENOSPACE
    assert call(T=1000) == lynx.LYNX_EINVAL
    assert call(Hq=34) == lynx.LYNX_EUNSUPPORTED
    assert call(dt=7) == lynx.LYNX_EINVAL
    assert call(B=0) == lynx.LYNX_OK
