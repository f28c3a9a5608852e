"""The accuracy study run through the GPU path: vNMSE of the Lynx full and anchor-only
attention outputs (GPU encode, lynx_attn_verify over full codes, lynx_attn_anchor over the
anchor stream) against the exact float64 attention over the BF16 KV, compared with the
oracle's values stored in tests/golden/accuracy_vnmse.txt (same workload and seeds).

Bar: |vNMSE_gpu - vNMSE_oracle| <= 5% of vNMSE_oracle + 2e-7 (the GPU attention's own
float32 / float16 arithmetic adds ~1e-8 at most on this workload).
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx
from oracle import accuracy as acc
from oracle import lynx_oracle as o

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(__file__)


def load_maker():
    spec = importlib.util.spec_from_file_location("mk", os.path.join(HERE, "golden", "make_accuracy_table.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    return mk


def stored_ablation():
    out, section = {}, None
    for line in open(os.path.join(HERE, "golden", "accuracy_vnmse.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            section = line
            continue
        if section == "[ablation]" and not line.startswith("config"):
            name, full, anchor = [x.strip() for x in line.split("|")]
            out[name] = (float(full), float(anchor))
    return out


def stored_methods():
    out, section = {}, None
    for line in open(os.path.join(HERE, "golden", "accuracy_vnmse.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            section = line
            continue
        if section == "[methods]" and not line.startswith("method"):
            name, *vals = [x.strip() for x in line.split("|")]
            out[name] = [float(x) for x in vals]
    return out


def test_vnmse_through_the_gpu_path(gpu):
    mk = load_maker()
    k, v, q = mk.inputs()
    B, T, Hkv, M, Hq = mk.B, mk.T, mk.HKV, mk.M, mk.HQ
    P, C, alpha = 256, 64, 255.0
    print(f"[accuracy] encoding {B} x {T} tokens on the GPU", flush=True)
    kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
    vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
    ka, kr = lynx.encode(kt, P, C, alpha)
    va, vr = lynx.encode(vt, P, C, alpha)
    stored = stored_methods()
    K = o.bf16_bits_to_f64(k)
    V = o.bf16_bits_to_f64(v)
    for col, s in enumerate(mk.Q_SCALES):
        qb = mk.scaled(q, s)
        ref = acc.attention_outputs(qb, K, V, T)
        qt = torch.from_numpy(np.ascontiguousarray(qb).view(np.int16)).view(torch.bfloat16).cuda()
        full, _ = lynx.attn_verify(qt, ka, kr, va, vr, T, Hkv, P, C, alpha, out_dtype=torch.float32)
        anchor = torch.stack([lynx.attn_anchor(qt[:, m].contiguous(), ka, va, T, Hkv, P, C, alpha,
                                               out_dtype=torch.float32) for m in range(M)], dim=1)
        torch.cuda.synchronize()
        got = {"Lynx": acc.vnmse(full.cpu().numpy().astype(np.float64), ref),
               "Lynx-INT4": acc.vnmse(anchor.cpu().numpy().astype(np.float64), ref)}
        for name, val in got.items():
            want = stored[name][col]
            print(f"[accuracy] q x {s}: {name} vNMSE gpu {val:.4e} oracle {want:.4e}", flush=True)
            assert abs(val - want) <= 0.05 * want + 2e-7


@pytest.mark.parametrize("label,P,C,alpha", [("C=16", 256, 16, 255.0), ("C=32", 256, 32, 255.0),
                                             ("alpha=2000", 256, 64, 2000.0), ("P=512", 512, 64, 255.0)])
def test_ablation_rows_through_the_gpu_path(gpu, label, P, C, alpha):
    """Rows of the reviewer's ablation (chunk size, alpha, page size) at query scale 0.1: the GPU
    path's vNMSE for Lynx (full codes, verification kernel) and Lynx-INT4 (anchor attention)
    against the stored oracle values."""
    mk = load_maker()
    k, v, q = mk.inputs()
    T, Hkv, M = mk.T, mk.HKV, mk.M
    print(f"[accuracy] ablation {label}", flush=True)
    kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
    vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
    ka, kr = lynx.encode(kt, P, C, alpha)
    va, vr = lynx.encode(vt, P, C, alpha)
    qb = mk.scaled(q, mk.ABLATION_Q)
    ref = acc.attention_outputs(qb, o.bf16_bits_to_f64(k), o.bf16_bits_to_f64(v), T)
    qt = torch.from_numpy(np.ascontiguousarray(qb).view(np.int16)).view(torch.bfloat16).cuda()
    full, _ = lynx.attn_verify(qt, ka, kr, va, vr, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    anchor = torch.stack([lynx.attn_anchor(qt[:, m].contiguous(), ka, va, T, Hkv, P, C, alpha,
                                           out_dtype=torch.float32) for m in range(M)], dim=1)
    torch.cuda.synchronize()
    want_full, want_anchor = stored_ablation()[label]
    for name, val, want in (("Lynx", acc.vnmse(full.cpu().numpy().astype(np.float64), ref), want_full),
                            ("Lynx-INT4", acc.vnmse(anchor.cpu().numpy().astype(np.float64), ref), want_anchor)):
        print(f"[accuracy] {label} {name}: vNMSE gpu {val:.4e} oracle {want:.4e}", flush=True)
        assert abs(val - want) <= 0.05 * want + 2e-7
