"""Benchmark of the Lynx hot path on one MI355X: encode + anchor-only decode + full
decode of a Llama-3-8B-shaped request, and the fused anchor-only decode attention.

One step =
  encode        32 layers x {K, V} x 16384 tokens x 8 kv heads x 128 (BF16, 2.15 GB),
                P = 256, C = 64, alpha = 255, anchor + residual streams
  decode_anchor the same request back to BF16 from the anchor segments
  decode_full   the same request back to BF16 from anchor + residual
  attn_anchor   16 sequences x 64 query heads / 8 kv heads x 32768-token context
                over anchor segments (P = 256, C = 64, alpha = 255)
Inputs are synthetic (Laplacian + per-channel offset + x100 outlier channels,
seeded) and resident in HBM before the timed region.

Prints one JSON line (rank 0, N = 1).  value = BF16-equivalent KV bytes processed
per second over the whole step (2 B x elements x 4 ops) in GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LAYERS, TOKENS, KVH, D = 32, 16384, 8, 128
P, C, ALPHA = 256, 64, 255.0
AB, AHQ, AHKV, AT = 16, 64, 8, 32768
KERNEL_SOURCES = ["decode_attention_lynx_amd/csrc/lynx_codec.hip", "decode_attention_lynx_amd/csrc/lynx_attn.hip",
                  "decode_attention_lynx_amd/csrc/lynx_common.hpp", "decode_attention_lynx_amd/csrc/lynx_abi.hip"]


def alg_bytes_per_elem(op: str) -> float:
    """Algorithmic HBM bytes per KV element (BF16 in/out 2 B, codes 0.5 B per stream,
    float32 metadata 8/C + 8/P B)."""
    meta = 8.0 / C + 8.0 / P
    return {"encode": 2.0 + 1.0 + meta, "decode_anchor": 0.5 + meta + 2.0, "decode_full": 1.0 + meta + 2.0,
            "attn_anchor": 0.5 + meta, "copy": 4.0}[op]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/traffic.json),
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec or rec.get("source_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(budget_s: float = 15.0):
    """The float64 oracle on a bounded sample of the same workload, on this host."""
    import numpy as np
    from decode_attention_lynx_amd import synth
    from oracle import lynx_oracle as o
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:       # pragma: no cover
        limiter = None
    t_codec = 0.0
    elems = 0
    pages = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s * 0.7 and pages < 4096:
        bits = synth.make_kv_np(P, KVH, D, seed=0, layer=pages, kv_idx=0)
        s = time.perf_counter()
        anc, res, _ = o.encode(bits, P, C, ALPHA)
        o.decode_anchor(anc, 1, P, KVH, D, C, ALPHA)
        o.decode_full(anc, res, 1, P, KVH, D, C, ALPHA)
        t_codec += time.perf_counter() - s
        elems += P * KVH * D
        pages += 1
    # attention: one sequence, one kv head group, a context prefix of the benchmark shape
    T = 4096
    kb = synth.make_kv_np(T, AHKV, D, seed=0, layer=0, kv_idx=0)
    vb = synth.make_kv_np(T, AHKV, D, seed=0, layer=0, kv_idx=1)
    ka, _, _ = o.encode(kb, P, C, ALPHA)
    va, _, _ = o.encode(vb, P, C, ALPHA)
    qb = synth.make_q_np(1, AHQ, D, seed=0)
    s = time.perf_counter()
    o.attention_anchor(qb, ka, va, 1, T, AHQ, AHKV, D, P, C, ALPHA)
    t_attn = time.perf_counter() - s
    attn_elems = 2 * T * AHKV * D
    if limiter is not None:
        limiter.unregister()
    bf16_bytes = 2.0 * (3 * elems + attn_elems)
    return {"value": round(bf16_bytes / (t_codec + t_attn) / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 numpy oracle, 1 thread: encode+decode_anchor+decode_full of {pages} pages "
                      f"(256 tok x 8 kvh x 128) and anchor attention of 1 sequence x 64 q-heads over a "
                      f"{T}-token prefix; {t_codec + t_attn:.1f} s of CPU time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ops", default="encode,decode_anchor,decode_full,attn_anchor")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Lynx hot path here is single-GPU (the codec and the "
              "attention shard by page / sequence with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_lynx_amd import lynx, synth

    dev = torch.device("cuda:0")
    ops = args.ops.split(",")
    print(f"[bench] generating request {LAYERS}x2x{TOKENS}x{KVH}x{D} and attention inputs", file=sys.stderr,
          flush=True)
    T_all = LAYERS * 2 * TOKENS
    n_pages = T_all // P
    kv = torch.empty((T_all, KVH, D), dtype=torch.bfloat16, device=dev)
    for layer in range(LAYERS):
        for kv_idx in (0, 1):
            t0 = (layer * 2 + kv_idx) * TOKENS
            synth.make_kv_torch(TOKENS, KVH, D, seed=0, layer=layer, kv_idx=kv_idx, out=kv[t0:t0 + TOKENS])
    a_sz, r_sz = lynx.stream_sizes(P, KVH, D, C)
    anchor = torch.empty((n_pages, a_sz), dtype=torch.uint8, device=dev)
    residual = torch.empty((n_pages, r_sz), dtype=torch.uint8, device=dev)
    out_a = torch.empty_like(kv)
    out_f = torch.empty_like(kv)
    # attention inputs: anchor segments of 16 sequences x 32768 tokens, encoded once
    akv = torch.empty((AB * AT, AHKV, D), dtype=torch.bfloat16, device=dev)
    att = {}
    for kv_idx in (0, 1):
        for b in range(AB):
            synth.make_kv_torch(AT, AHKV, D, seed=1, layer=b, kv_idx=kv_idx, out=akv[b * AT:(b + 1) * AT])
        att[kv_idx], _ = lynx.encode(akv, P, C, ALPHA, residual=False)
    del akv
    q = synth.make_q_torch(AB, AHQ, D, seed=0)
    ws = torch.empty(lynx.attn_workspace_bytes(AB, AT, AHQ, AHKV, D, P, C), dtype=torch.uint8, device=dev)
    o_att = torch.empty((AB, AHQ, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    copy_src = copy_dst = None
    if "copy" in ops:       # plain 1 GiB device copy: calibrates the HBM byte counters
        copy_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    def run(op):
        if op == "copy":
            copy_dst.copy_(copy_src)
        elif op == "encode":
            lynx.encode(kv, P, C, ALPHA, anchor_out=anchor, residual_out=residual)
        elif op == "decode_anchor":
            lynx.decode_anchor(anchor, n_pages, P, KVH, D, C, ALPHA, out=out_a)
        elif op == "decode_full":
            lynx.decode_full(anchor, residual, n_pages, P, KVH, D, C, ALPHA, out=out_f)
        elif op == "attn_anchor":
            lynx.attn_anchor(q, att[0], att[1], AT, AHKV, P, C, ALPHA, workspace=ws, out=o_att)

    elems = {"encode": T_all * KVH * D, "decode_anchor": T_all * KVH * D, "decode_full": T_all * KVH * D,
             "attn_anchor": 2 * AB * AT * AHKV * D, "copy": (1 << 30) // 2}
    for _ in range(args.warmup):
        for op in ops:
            run(op)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = {op: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for op in ops}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for op in ops:
            ev[op][s][0].record(stream)
            run(op)
            ev[op][s][1].record(stream)
        print(f"[bench] step {s + 1}/{args.steps} enqueued", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {op: sum(a.elapsed_time(b) for a, b in ev[op]) / args.steps for op in ops}
    step_ms = wall * 1e3 / args.steps
    per_op = {}
    for op in ops:
        alg = alg_bytes_per_elem(op) * elems[op]
        per_op[op] = {"ms": round(ms[op], 4), "bf16_equiv_GBs": round(2.0 * elems[op] / ms[op] / 1e6, 1),
                      "alg_GBs": round(alg / ms[op] / 1e6, 1), "frac_hbm_peak": round(alg / ms[op] / 1e6 / HBM_PEAK_GBS, 4),
                      "alg_bytes_per_launch": int(alg)}
    path_ops = [op for op in ops if op != "copy"]
    total_bf16 = sum(2.0 * elems[op] for op in path_ops)
    value = total_bf16 / (step_ms / 1e3) / 1e9
    dom = max(path_ops or ops, key=lambda o_: ms[o_])
    achieved = per_op[dom]["alg_GBs"]
    rec = {
        "metric": "KV GB/s (BF16-equiv) encode/decode + anchor-attn, % of MI355X HBM peak",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3-8b request codec (32 layers x K,V x 16384 tok x 8 kvh x 128 BF16, P=256, "
                               "C=64, alpha=255: encode + decode_anchor + decode_full) + anchor-only decode "
                               "attention (16 seq x 64 q / 8 kv heads x 128, 32768-token context)",
                   "ops": per_op, "hbm_peak_GBs": HBM_PEAK_GBS,
                   "arith": "float32 codec (float64 statistics and boundary cases), float16 MFMA attention "
                            "with float32 accumulation"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(dom)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
