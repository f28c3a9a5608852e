"""GPU parity of the fused anchor-only decode attention against the oracle.

The oracle (float64) decodes the same anchor segments and evaluates Eq. 1 of
the technical review (softmax(q K^T / sqrt(d)) V) per query head.  Bar:
relative L2 of the whole output <= 2e-3 (float32 output), and the error of every
query head <= 1e-2 of the root-mean-square head norm of the case (so an error local to one
head cannot hide under the global norm; a head whose own output is small because its values
cancel is not held to its own norm, which float16 operands cannot resolve).  Small cases use oracle-encoded codes uploaded to the GPU, so the
attention is checked independently of the GPU encoder; the full-size case
(16 sequences x 32768 tokens) uses GPU-encoded codes and samples sequences.
"""
import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth
from oracle import lynx_oracle as o

pytestmark = pytest.mark.gpu
REL_L2 = 2e-3
HEAD_L2 = 1e-2          # per (sequence, query head), relative to the RMS head norm


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def worst_head(got, ref):
    """Largest per-head error over the RMS head norm, and over the head's own norm."""
    err = np.linalg.norm(got - ref, axis=-1)
    norm = np.linalg.norm(ref, axis=-1)
    rms = float(np.sqrt(np.mean(norm ** 2)))
    return float(err.max() / rms), float((err / np.maximum(norm, 1e-300)).max())


def check(got, ref, tag):
    e = rel_l2(got, ref)
    w, w_own = worst_head(got, ref)
    print(f"[attn] {tag}: rel_l2={e:.3e} worst_head={w:.3e} (own norm {w_own:.3e})", flush=True)
    assert e <= REL_L2
    assert w <= HEAD_L2


def upload(u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u8)).cuda()


def make_case(B, Hq, Hkv, T, P, C, alpha, seed):
    kb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=seed, layer=b, kv_idx=0) for b in range(B)])
    vb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=seed, layer=b, kv_idx=1) for b in range(B)])
    ka, _, _ = o.encode(kb, P, C, alpha)
    va, _, _ = o.encode(vb, P, C, alpha)
    qb = synth.make_q_np(B, Hq, 128, seed=seed)
    return qb, ka, va


@pytest.mark.parametrize("B,Hq,Hkv,T,P,C,alpha", [
    (2, 16, 2, 1024, 256, 64, 255.0),
    (3, 8, 1, 320, 64, 64, 255.0),       # 5 pages of 64 tokens: ragged split of tiles
    (2, 12, 4, 512, 256, 128, 63.0),     # group of 3 query heads, chunk of 128
    (1, 2, 2, 64, 64, 64, 15.0),         # one tile, group of 1
    (1, 64, 8, 2048, 256, 64, 255.0),    # the full head geometry, short context
    (2, 16, 2, 1024, 256, 32, 255.0),    # chunk of 32 (the pages' own setting): two chunks per 64-token tile
    (1, 8, 1, 96, 32, 32, 63.0),         # chunk 32, three pages of one chunk each
    (1, 16, 2, 8192, 4096, 256, 255.0),  # two 4096-token pages, chunks of 256 (four tiles each)
    (2, 16, 2, 1024, 256, 16, 255.0),    # chunk of 16: four chunks per 64-token tile
    (1, 8, 1, 512, 64, 16, 63.0),        # chunk of 16 in 64-token pages
    (2, 16, 2, 1024, 256, 8, 255.0),     # chunk of 8: four chunks per 32-token tile
    (1, 8, 1, 96, 32, 8, 15.0),          # chunk of 8, three 32-token pages
    (2, 32, 2, 1024, 256, 64, 255.0),    # group of 16 query heads (one MFMA column per head)
    (1, 48, 4, 512, 256, 32, 255.0),     # group of 12, two chunks of 32 per tile
    (1, 64, 4, 1024, 256, 16, 255.0),    # group of 16, chunk of 16
    (1, 16, 1, 512, 256, 8, 255.0),      # group of 16, chunk of 8
    (32, 8, 8, 1536, 96, 32, 255.0),     # 32-token tiles of one chunk; every wave walks four tiles
])
def test_attention_small(gpu, B, Hq, Hkv, T, P, C, alpha):
    print(f"[attn] B={B} Hq={Hq} Hkv={Hkv} T={T} P={P} C={C} alpha={alpha}", flush=True)
    qb, ka, va = make_case(B, Hq, Hkv, T, P, C, alpha, seed=T + Hq)
    ref = o.attention_anchor(qb, ka, va, B, T, Hq, Hkv, 128, P, C, alpha)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
    k, v = upload(ka), upload(va)
    out32 = lynx.attn_anchor(q, k, v, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    out16 = lynx.attn_anchor(q, k, v, T, Hkv, P, C, alpha, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out32.cpu().numpy().astype(np.float64)
    check(got, ref, "small")
    # the BF16 output is the float32 result rounded to nearest even
    g16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(g16, o.f64_to_bf16_bits(out32.cpu().numpy().astype(np.float64)))


def test_attention_sm_scale_argument(gpu):
    """sm_scale > 0 replaces 1/sqrt(128)."""
    B, Hq, Hkv, T, P, C = 1, 8, 1, 256, 256, 64
    qb, ka, va = make_case(B, Hq, Hkv, T, P, C, 255.0, seed=11)
    ref = o.attention_anchor(qb, ka, va, B, T, Hq, Hkv, 128, P, C, 255.0, sm_scale=0.02)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
    out = lynx.attn_anchor(q, upload(ka), upload(va), T, Hkv, P, C, 255.0, sm_scale=0.02)
    torch.cuda.synchronize()
    check(out.cpu().numpy().astype(np.float32).astype(np.float64), ref, "sm_scale")


def test_attention_full_size_sampled(gpu):
    """16 sequences x 64 query heads / 8 kv heads x 32768 tokens, P=256, C=64, alpha=255, in
    the launch configuration the benchmark times; the oracle checks three sequences."""
    B, Hq, Hkv, T, P, C, alpha = 16, 64, 8, 32768, 256, 64, 255.0
    print("[attn] full size: generating and encoding K/V on the GPU", flush=True)
    kv = torch.empty((B * T, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    ka, va = [], []
    for kv_idx in (0, 1):
        for b in range(B):
            synth.make_kv_torch(T, Hkv, 128, seed=0, layer=b, kv_idx=kv_idx, out=kv[b * T:(b + 1) * T])
        anc, _ = lynx.encode(kv, P, C, alpha, residual=False)
        (ka if kv_idx == 0 else va).append(anc)
    ka, va = ka[0], va[0]
    q = synth.make_q_torch(B, Hq, 128, seed=0)
    out = lynx.attn_anchor(q, ka, va, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    npg = T // P
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    KA, VA = ka.cpu().numpy(), va.cpu().numpy()
    got = out.cpu().numpy().astype(np.float64)
    for b in (0, 7, 15):
        print(f"[attn] oracle on sequence {b}", flush=True)
        ref = o.attention_anchor(qb[b:b + 1], KA[b * npg:(b + 1) * npg], VA[b * npg:(b + 1) * npg], 1, T, Hq,
                                 Hkv, 128, P, C, alpha)
        check(got[b:b + 1], ref, f"full size, seq {b}")


@pytest.mark.parametrize("C", [64, 32, 16])
def test_attention_paged_variable_lengths(gpu, C):
    """A shuffled pool of pages behind a block table, with lengths that end inside a tile, on a
    tile edge, inside a page, at one token and at zero (output 0)."""
    B, Hq, Hkv, P, maxp, alpha = 6, 16, 2, 256, 4, 255.0
    lens = np.array([1, 63, 64, 300, maxp * P, 0], dtype=np.int32)
    print(f"[attn-paged] C={C} lens={lens.tolist()}", flush=True)
    T = maxp * P
    kb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=31, layer=b, kv_idx=0) for b in range(B)])
    vb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=31, layer=b, kv_idx=1) for b in range(B)])
    ka, _, _ = o.encode(kb, P, C, alpha)
    va, _, _ = o.encode(vb, P, C, alpha)
    perm = np.random.default_rng(C).permutation(B * maxp)
    inv = np.argsort(perm)
    bt = inv[np.arange(B * maxp).reshape(B, maxp)].astype(np.int32)
    bt[0, 1:] = -1                                   # pages past a sequence's end are not read
    qb = synth.make_q_np(B, Hq, 128, seed=31)
    ref = o.attention_anchor_paged(qb, ka[perm], va[perm], bt, lens, Hq, Hkv, 128, P, C, alpha)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
    out = lynx.attn_anchor_paged(q, upload(ka[perm]), upload(va[perm]), torch.from_numpy(bt).cuda(),
                                 torch.from_numpy(lens).cuda(), Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0)
            continue
        check(got[b:b + 1], ref[b:b + 1], f"paged seq {b} len {lens[b]}")


def test_attention_group_of_16_long_context(gpu):
    """The long-context model's geometry: 64 query heads over 4 kv heads (a group of 16), one
    sequence of 32768 tokens, encoded on the GPU."""
    B, Hq, Hkv, T, P, C, alpha = 1, 64, 4, 32768, 256, 64, 255.0
    kv = [torch.empty((T, Hkv, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for kv_idx in (0, 1):
        synth.make_kv_torch(T, Hkv, 128, seed=9, layer=0, kv_idx=kv_idx, out=kv[kv_idx])
    ka, _ = lynx.encode(kv[0], P, C, alpha, residual=False)
    va, _ = lynx.encode(kv[1], P, C, alpha, residual=False)
    q = synth.make_q_torch(B, Hq, 128, seed=9)
    out = lynx.attn_anchor(q, ka, va, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = o.attention_anchor(qb, ka.cpu().numpy(), va.cpu().numpy(), B, T, Hq, Hkv, 128, P, C, alpha)
    check(out.cpu().numpy().astype(np.float64), ref, "group 16, 32768 tokens")


@pytest.mark.parametrize("key_scale,C,soft", [(3e4, 64, True), (3e4, 16, False), (1e12, 32, False)])
def test_attention_keys_beyond_float16_range(gpu, key_scale, C, soft):
    """Key channels of range ~1e5 (and ~1e13): the folded query q * (gamma_scale + eps)(sigma +
    eps) * scale leaves the float16 range, so the kernel carries it with a power-of-two exponent.
    Values are scaled the same way on other channels.  With `soft` the query components on the
    huge channels are scaled down so the softmax stays soft (the exponent is still taken, from
    the bound); otherwise those channels decide the scores.  The outputs must match the oracle."""
    B, Hq, Hkv, T, P, alpha = 2, 16, 2, 1024, 256, 255.0
    rng = np.random.default_rng(int(np.log10(key_scale)) + C)
    kx = rng.laplace(0, 0.5, size=(B * T, Hkv, 128))
    vx = rng.laplace(0, 0.5, size=(B * T, Hkv, 128))
    kx[:, :, 5] *= key_scale                          # one huge key channel per head
    kx[:, 1, 77] *= key_scale / 7                     # and a second one in head 1
    vx[:, :, 9] *= key_scale                          # values beyond float16 as well
    kb, vb = o.f64_to_bf16_bits(kx), o.f64_to_bf16_bits(vx)
    ka, _, _ = o.encode(kb, P, C, alpha)
    va, _, _ = o.encode(vb, P, C, alpha)
    qb = synth.make_q_np(B, Hq, 128, seed=4)
    if soft:     # the huge channels enter the scores through small query components
        q64 = o.bf16_bits_to_f64(qb)
        q64[:, :, 5] *= 1.0 / key_scale
        q64[:, :, 77] *= 1.0 / key_scale
        qb = o.f64_to_bf16_bits(q64)
    ref = o.attention_anchor(qb, ka, va, B, T, Hq, Hkv, 128, P, C, alpha)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
    out = lynx.attn_anchor(q, upload(ka), upload(va), T, Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(out.cpu().numpy().astype(np.float64), ref, f"keys x{key_scale:g}, C={C}, soft={soft}")
