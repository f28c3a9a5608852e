"""Full-size GPU parity of the codec on the request shapes, in the launch
configuration the benchmark times, checked against the oracle on sampled pages.

  * Llama-3-8B request: 32 layers x {K, V} x 16384 tokens x 8 kv heads x 128,
    one encode call over all 4096 pages (as timed), both decoders.
  * Qwen-32B request: 64 layers x {K, V} x 16384 x 8 x 128, the chunk / alpha
    sweep C in {32, 64, 128} x alpha in {15, 63, 255}, one call per setting.
  * Qwen3-235B long context: 94 layers x {K, V} x 131072 tokens x 4 kv heads x
    128, resident in HBM (25 GB) and streamed one layer tensor per call.

Inputs are drawn on the GPU (same recipe as the small cases); sampled pages are
copied back and checked element by element under the contract of tests/parity.py.
"""
import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth
from oracle import lynx_oracle as o
from tests import parity

pytestmark = pytest.mark.gpu
P = 256


def check_pages(kv, anc, res, pages, C, alpha, Hkv, label, dec_f32=None, dec_bf16=None):
    """kv: device BF16 [n_pages*P, Hkv, 128]; anc/res: device segments; pages: indices to check.
    dec_f32 / dec_bf16: optional dicts name -> device decode outputs over the same pages."""
    rep = {}
    H = Hkv * 128
    for p in pages:
        bits = kv[p * P:(p + 1) * P].view(torch.int16).cpu().numpy().view(np.uint16)
        X = o.bf16_bits_to_f64(bits).reshape(P, H)
        A = anc[p].cpu().numpy()
        got = o.parse_anchor_segment(A, P, Hkv, 128, C)
        enc = o.encode_page(X, C, alpha)
        q_res = o.unpack_nibbles(res[p].cpu().numpy(), P, Hkv, 128)
        parity.check_metadata(got, enc, X, C, rep)
        parity.check_codes(got, q_res, X, C, alpha, rep)
        args = (got["mu"], got["sigma"], got["gmin"], got["gscale"], C, alpha)
        refs = {"anchor": o.decode_page_anchor(got["Q_anc"], *args),
                "full": o.decode_page_full(got["Q_anc"], q_res, *args)}
        sl = slice(p * P, (p + 1) * P)
        for name, out in (dec_f32 or {}).items():
            parity.check_decode_f32(out[sl].cpu().numpy().reshape(P, H), refs[name], got["gscale"], rep)
        for name, out in (dec_bf16 or {}).items():
            parity.check_decode_bf16(out[sl].view(torch.int16).cpu().numpy().view(np.uint16).reshape(P, H),
                                     refs[name], parity.decode_slack(got, refs[name], C), rep)
    parity.finish_codes(rep)
    if dec_bf16:
        parity.finish_bf16(rep)
    print(f"[full] {label}: {rep}", flush=True)


def make_request(layers, tokens, Hkv, seed=0):
    kv = torch.empty((layers * 2 * tokens, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    for layer in range(layers):
        for kv_idx in (0, 1):
            t0 = (layer * 2 + kv_idx) * tokens
            synth.make_kv_torch(tokens, Hkv, 128, seed=seed, layer=layer, kv_idx=kv_idx, out=kv[t0:t0 + tokens])
    return kv


def sample_pages(n_pages, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, n_pages - 1] + rng.choice(n_pages, size=k, replace=False).tolist()))


def test_llama3_8b_request_full_size(gpu):
    print("[full] llama3-8b request: 32 x 2 x 16384 x 8 x 128", flush=True)
    kv = make_request(32, 16384, 8)
    n_pages = kv.shape[0] // P
    anc, res = lynx.encode(kv, P, 64, 255.0)
    da16 = lynx.decode_anchor(anc, n_pages, P, 8, 128, 64, 255.0)
    df16 = lynx.decode_full(anc, res, n_pages, P, 8, 128, 64, 255.0)
    df32 = lynx.decode_full(anc, res, n_pages, P, 8, 128, 64, 255.0, out_dtype=torch.float32)
    da32 = lynx.decode_anchor(anc, n_pages, P, 8, 128, 64, 255.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_pages(kv, anc, res, sample_pages(n_pages, 10, 1), 64, 255.0, 8, "llama3-8b C64 a255",
                dec_f32={"anchor": da32, "full": df32}, dec_bf16={"anchor": da16, "full": df16})


@pytest.mark.parametrize("C", [32, 64, 128])
def test_qwen32b_request_chunk_alpha_sweep(gpu, C):
    print(f"[full] qwen-32b request: 64 x 2 x 16384 x 8 x 128, C={C}", flush=True)
    kv = make_request(64, 16384, 8, seed=2)
    n_pages = kv.shape[0] // P
    for alpha in (15.0, 63.0, 255.0):
        anc, res = lynx.encode(kv, P, C, alpha)
        df32 = lynx.decode_full(anc, res, n_pages, P, 8, 128, C, alpha, out_dtype=torch.float32)
        da32 = lynx.decode_anchor(anc, n_pages, P, 8, 128, C, alpha, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_pages(kv, anc, res, sample_pages(n_pages, 3, C + int(alpha)), C, alpha, 8,
                    f"qwen-32b C{C} a{alpha:g}", dec_f32={"anchor": da32, "full": df32})
        del anc, res, df32, da32


def test_qwen3_235b_long_context_streamed(gpu):
    """25 GB of KV resident in HBM, encoded and decoded one layer tensor (512 pages) per call."""
    L, T, Hkv, C, alpha = 94, 131072, 4, 64, 255.0
    print("[full] qwen3-235b long context: 94 x 2 x 131072 x 4 x 128 (25.2 GB)", flush=True)
    kv = make_request(L, T, Hkv, seed=3)
    pages_per_tensor = T // P
    a_sz, r_sz = lynx.stream_sizes(P, Hkv, 128, C)
    anc = torch.empty((pages_per_tensor, a_sz), dtype=torch.uint8, device="cuda")
    res = torch.empty((pages_per_tensor, r_sz), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, Hkv, 128), dtype=torch.float32, device="cuda")
    for tensor in range(2 * L):
        part = kv[tensor * T:(tensor + 1) * T]
        lynx.encode(part, P, C, alpha, anchor_out=anc, residual_out=res)
        if tensor % 47 == 0 or tensor == 2 * L - 1:
            lynx.decode_full(anc, res, pages_per_tensor, P, Hkv, 128, C, alpha, out=out)
            torch.cuda.synchronize()
            print(f"[full] layer tensor {tensor}", flush=True)
            check_pages(part, anc, res, sample_pages(pages_per_tensor, 2, tensor), C, alpha, Hkv,
                        f"qwen3-235b tensor {tensor}", dec_f32={"full": out})
    torch.cuda.synchronize()
