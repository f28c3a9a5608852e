"""The anchor attention's no-allocation entry point (lynx_attn_anchor_noalloc), called through the
C ABI, against the entry point with a caller workspace (lynx_attn_anchor) on the same inputs: the
same kernels and the same record layout, so the outputs must be identical.  Two calls in a row on
the library's per-GPU buffer, the second with a smaller input, then the first shape again; and a
shape whose partial results exceed the buffer is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth

pytestmark = pytest.mark.gpu


def encode_case(B, Hkv, T, P, C, seed):
    kv = torch.empty((B * T, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    segs = []
    for kv_idx in (0, 1):
        for b in range(B):
            synth.make_kv_torch(T, Hkv, 128, seed=seed, layer=b, kv_idx=kv_idx, out=kv[b * T:(b + 1) * T])
        anc, _ = lynx.encode(kv, P, C, 255.0, residual=False)
        segs.append(anc)
    return segs


def call_noalloc(q, ka, va, T, Hkv, P, C, out):
    B, Hq, D = q.shape
    st = lynx.lib().lynx_attn_anchor_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(ka.data_ptr()), ctypes.c_void_p(va.data_ptr()), B, T, Hq,
        Hkv, D, P, C, 255.0, 0.0, lynx.OUT_F32, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == lynx.LYNX_OK, lynx.strerror(st)


def test_noalloc_matches_workspace_entry_point(gpu):
    cases = [(16, 64, 8, 32768, 256, 64, 1), (2, 16, 2, 1024, 256, 32, 2), (16, 64, 8, 32768, 256, 64, 1)]
    for B, Hq, Hkv, T, P, C, seed in cases:
        print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} T={T} P={P} C={C}", flush=True)
        ka, va = encode_case(B, Hkv, T, P, C, seed)
        q = synth.make_q_torch(B, Hq, 128, seed=seed)
        ref = lynx.attn_anchor(q, ka, va, T, Hkv, P, C, 255.0, out_dtype=torch.float32)
        out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        call_noalloc(q, ka, va, T, Hkv, P, C, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), float((out - ref).abs().max())
        # the binding's wrapper of the same entry point
        out2 = lynx.attn_anchor_noalloc(q, ka, va, T, Hkv, P, C, 255.0)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_refuses_shapes_beyond_its_buffer(gpu):
    # 1024 sequences x 64 query heads: one (m, l, o[128]) record per head and split, 34 MB
    B, Hq, Hkv, T, P, C = 1024, 64, 8, 256, 256, 64
    need = lynx.attn_workspace_bytes(B, T, Hq, Hkv, 128, P, C)
    assert need > lynx.ATTN_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    st = lynx.lib().lynx_attn_anchor_noalloc(p, p, p, B, T, Hq, Hkv, 128, P, C, 255.0, 0.0, lynx.OUT_F32, p, None)
    assert st == lynx.LYNX_ENOSPACE
