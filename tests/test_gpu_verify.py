"""GPU parity of the verification-pass attention over full codes against the oracle.

The oracle (float64) decodes the same anchor + residual segments with the full
decoder and evaluates Eq. 1 of the technical review for every draft token and
query head, with the natural-log log-sum-exp of the scaled scores.  Bars:
relative L2 of the whole output <= 2e-3 (float32 output); the LSE within the
error of the kernel's key format (see lse_bound).  Small cases use
oracle-encoded codes uploaded to the GPU; the
full-size case (16 sequences x 64 draft tokens x 32768 context tokens) uses
GPU-encoded codes and checks sampled sequences.
"""
import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth
from oracle import lynx_oracle as o

pytestmark = pytest.mark.gpu
REL_L2 = 2e-3
ROW_L2 = 1e-2           # per (sequence, draft token, query head) row, relative to the RMS row norm


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def upload(u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u8)).cuda()


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def make_case(B, M, Hq, Hkv, T, P, C, alpha, seed):
    kb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=seed, layer=b, kv_idx=0) for b in range(B)])
    vb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=seed, layer=b, kv_idx=1) for b in range(B)])
    ka, kr, _ = o.encode(kb, P, C, alpha)
    va, vr, _ = o.encode(vb, P, C, alpha)
    qb = synth.make_q_np(B * M, Hq, 128, seed=seed).reshape(B, M, Hq, 128)
    return qb, ka, kr, va, vr


def lse_bound(qb, ka, kr, B, M, T, Hq, Hkv, P, C, alpha, sm_scale=None):
    """Per (sequence, draft token, query head) bound on |lse_gpu - lse_oracle|.

    The kernel carries each decoded key as a BF16 high part plus a BF16 low part, both rounded to
    nearest (8 significant bits, unit roundoff 2^-8): |k - hi - lo| <= 2^-8 |k - hi| <= 2^-16 |k|.
    A score then errs by at most 2^-16 * scale * sum_d |q_d k_d| (plus float32 rounding of the key
    and of the sum, covered by doubling the factor), and the LSE by at most the largest score error
    of its row; 2e-6 relative covers the float32 exp2 / log2 of the reduction."""
    scale = 1.0 / np.sqrt(128) if sm_scale is None else sm_scale
    G = Hq // Hkv
    npg = T // P
    q = np.abs(o.bf16_bits_to_f64(qb))
    out = np.empty((B, M, Hq))
    for b in range(B):
        K = np.abs(o.decode_full(ka[b * npg:(b + 1) * npg].reshape(-1), kr[b * npg:(b + 1) * npg].reshape(-1), npg,
                                 P, Hkv, 128, C, alpha))
        for h in range(Hkv):
            qg = q[b, :, h * G:(h + 1) * G, :].reshape(M * G, 128)
            out[b, :, h * G:(h + 1) * G] = (qg @ K[:, h, :].T).max(axis=1).reshape(M, G)
    return 2.0 ** -15 * scale * out


def check(got_o, got_lse, ref_o, ref_lse, bound, tag):
    e = rel_l2(got_o, ref_o)
    err = np.linalg.norm(got_o - ref_o, axis=-1)
    worst = float(err.max() / np.sqrt(np.mean(np.linalg.norm(ref_o, axis=-1) ** 2)))
    de = np.abs(got_lse - ref_lse)
    tol = bound + 2e-6 * (1.0 + np.abs(ref_lse))
    print(f"[verify] {tag}: rel_l2={e:.3e} worst_row={worst:.3e} lse_max_abs={de.max():.3e} "
          f"worst lse err / bound={float((de / tol).max()):.3f}", flush=True)
    assert e <= REL_L2
    assert worst <= ROW_L2
    assert np.all(de <= tol)


@pytest.mark.parametrize("B,M,Hq,Hkv,T,P,C,alpha", [
    (2, 4, 16, 2, 1024, 256, 64, 255.0),    # 32 query rows per kv head: one partly used row block
    (1, 16, 64, 8, 512, 256, 64, 255.0),    # exactly one block of 128 rows
    (1, 17, 64, 8, 256, 256, 64, 255.0),    # 136 rows: a second, ragged row block
    (3, 1, 8, 1, 320, 64, 64, 255.0),       # one draft token; 5 pages of 64 tokens
    (2, 5, 12, 4, 512, 256, 128, 63.0),     # group of 3 query heads, chunk of 128
    (1, 64, 64, 8, 2048, 256, 64, 255.0),   # 64 draft tokens, the full head geometry
    (1, 3, 2, 2, 64, 64, 64, 15.0),         # one tile, group of 1
    (2, 4, 16, 2, 1024, 256, 32, 255.0),    # chunk of 32 (the pages' own setting): two chunks per tile
    (1, 9, 24, 4, 384, 64, 32, 63.0),       # chunk 32 in one-tile pages, group of 6, 54 rows
    (1, 4, 16, 2, 8192, 4096, 256, 63.0),   # two 4096-token pages, chunks of 256 (four tiles each)
    (2, 4, 16, 2, 1024, 256, 16, 255.0),    # chunk of 16: four chunks per tile
    (1, 3, 8, 1, 192, 64, 16, 15.0),        # chunk of 16 in 64-token pages
    (1, 4, 64, 4, 1024, 256, 64, 255.0),    # group of 16 query heads (64 q / 4 kv heads)
    (1, 2, 64, 4, 1024, 256, 16, 255.0),    # group of 16, chunk of 16
])
def test_verify_small(gpu, B, M, Hq, Hkv, T, P, C, alpha):
    print(f"[verify] B={B} M={M} Hq={Hq} Hkv={Hkv} T={T} P={P} C={C} alpha={alpha}", flush=True)
    qb, ka, kr, va, vr = make_case(B, M, Hq, Hkv, T, P, C, alpha, seed=T + M)
    ref_o, ref_lse = o.attention_verify(qb, ka, kr, va, vr, B, M, T, Hq, Hkv, 128, P, C, alpha)
    q = bf16_tensor(qb)
    args = (q, upload(ka), upload(kr), upload(va), upload(vr), T, Hkv, P, C, alpha)
    out32, lse = lynx.attn_verify(*args, out_dtype=torch.float32)
    out16, lse16 = lynx.attn_verify(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out32.cpu().numpy().astype(np.float64)
    bound = lse_bound(qb, ka, kr, B, M, T, Hq, Hkv, P, C, alpha)
    check(got, lse.cpu().numpy().astype(np.float64), ref_o, ref_lse, bound, "small")
    # the BF16 output is the float32 result rounded to nearest even; the LSE does not depend on it
    g16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(g16, o.f64_to_bf16_bits(out32.cpu().numpy().astype(np.float64)))
    assert torch.equal(lse, lse16)


def test_verify_without_lse_and_sm_scale(gpu):
    """lse may be omitted; sm_scale > 0 replaces 1/sqrt(128)."""
    B, M, Hq, Hkv, T, P, C = 1, 8, 8, 1, 256, 256, 64
    qb, ka, kr, va, vr = make_case(B, M, Hq, Hkv, T, P, C, 255.0, seed=5)
    ref_o, ref_lse = o.attention_verify(qb, ka, kr, va, vr, B, M, T, Hq, Hkv, 128, P, C, 255.0, sm_scale=0.02)
    args = (bf16_tensor(qb), upload(ka), upload(kr), upload(va), upload(vr), T, Hkv, P, C, 255.0)
    out, none = lynx.attn_verify(*args, sm_scale=0.02, want_lse=False)
    out2, lse = lynx.attn_verify(*args, sm_scale=0.02)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out, out2)
    bound = lse_bound(qb, ka, kr, B, M, T, Hq, Hkv, P, C, 255.0, sm_scale=0.02)
    check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_lse, bound,
          "sm_scale")


@pytest.mark.parametrize("factor", [4096.0, 128.0])
def test_verify_values_beyond_float16_range(gpu, factor):
    """Values the kernel cannot hold as float16 (|V| up to ~2*10^6 from token 1088 on at a factor
    of 4096; ~8*10^4 at 128, where several pages' bound |A_V| + |B_V| falls between 60000 and
    2^16, the edge of the exponent's first step) take its power-of-two range exponent.  With 8
    sequences of 32 one-tile pages the context splits hold 2 tiles each, so the exponent grows
    inside a split (tiles 16 -> 17); the bar is unchanged."""
    B, M, Hq, Hkv, T, P, C, alpha = 8, 4, 16, 2, 2048, 64, 64, 255.0
    kb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=21, layer=b, kv_idx=0) for b in range(B)])
    vf = np.concatenate([o.bf16_bits_to_f64(synth.make_kv_np(T, Hkv, 128, seed=21, layer=b, kv_idx=1))
                         for b in range(B)]).reshape(B, T, Hkv, 128)
    vf[:, 17 * 64:] *= factor                  # a power of two: the BF16 values stay exact
    assert np.abs(vf).max() > 65504.0
    vb = o.f64_to_bf16_bits(vf.reshape(B * T, Hkv, 128))
    ka, kr, _ = o.encode(kb, P, C, alpha)
    va, vr, pages = o.encode(vb, P, C, alpha)
    # the pages' bound on |V_hat| (|A_V| + |B_V| over their chunks and channels)
    bound = np.array([(np.abs((pg["gscale"] + 1e-6) * (pg["sigma"] + 1e-6)) +
                       np.abs(pg["gmin"] + pg["mu"] * (pg["gscale"] + 1e-6))).max() for pg in pages])
    assert np.any(bound > 65536.0)
    if factor == 128.0:
        assert np.any((bound > 60000.0) & (bound < 65536.0))
    qb = synth.make_q_np(B * M, Hq, 128, seed=21).reshape(B, M, Hq, 128)
    ref_o, ref_lse = o.attention_verify(qb, ka, kr, va, vr, B, M, T, Hq, Hkv, 128, P, C, alpha)
    out, lse = lynx.attn_verify(bf16_tensor(qb), upload(ka), upload(kr), upload(va), upload(vr), T, Hkv, P, C,
                                alpha)
    torch.cuda.synchronize()
    bound = lse_bound(qb, ka, kr, B, M, T, Hq, Hkv, P, C, alpha)
    check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_lse, bound,
          "range")


def test_verify_scores_rising_inside_splits(gpu):
    """Keys grow by 1.6x per tile inside each context split (8 sequences x 8 kv heads make 4 splits
    of 4 tiles), so a row's maximum rises tile after tile: some rises stay within what the kernel's
    probabilities absorb without moving its running maximum (below 8 in base 2), some may or may not
    (8 to 12: a lane's probabilities then sum to 2^12 or not), others move it (above 12); the
    inputs are checked to hold all three kinds.  Same bars as the small cases."""
    B, M, Hq, Hkv, T, P, C, alpha = 8, 2, 16, 8, 1024, 256, 64, 255.0
    npg, G = T // P, Hq // Hkv
    kf = np.concatenate([o.bf16_bits_to_f64(synth.make_kv_np(T, Hkv, 128, seed=33, layer=b, kv_idx=0))
                         for b in range(B)]).reshape(B, T, Hkv, 128)
    kf *= (1.6 ** ((np.arange(T) // 64) % 4))[None, :, None, None]
    kb = o.f64_to_bf16_bits(kf.reshape(B * T, Hkv, 128))
    vb = np.concatenate([synth.make_kv_np(T, Hkv, 128, seed=33, layer=b, kv_idx=1) for b in range(B)])
    ka, kr, _ = o.encode(kb, P, C, alpha)
    va, vr, _ = o.encode(vb, P, C, alpha)
    qb = synth.make_q_np(B * M, Hq, 128, seed=33).reshape(B, M, Hq, 128)
    # the kernel's plan: 4 context splits of 4 tiles
    ws = lynx.attn_verify_workspace_bytes(B, M, T, Hq, Hkv, 128, P, C)
    assert ws == B * M * Hq * 4 * 132 * 4
    # each row's tile maximum against the running maximum of the tiles before it in its split (base 2)
    q = o.bf16_bits_to_f64(qb)
    to_base2 = np.log2(np.e) / np.sqrt(128)
    rises = []
    for b in range(B):
        K = o.decode_full(ka[b * npg:(b + 1) * npg].reshape(-1), kr[b * npg:(b + 1) * npg].reshape(-1), npg, P,
                          Hkv, 128, C, alpha)
        for h in range(Hkv):
            s = (q[b, :, h * G:(h + 1) * G, :].reshape(M * G, 128) @ K[:, h, :].T) * to_base2
            tmax = s.reshape(M * G, T // 64, 64).max(axis=2)
            for sp in range(4):
                run = tmax[:, 4 * sp]
                for j in range(1, 4):
                    rises.append(tmax[:, 4 * sp + j] - run)
                    run = np.maximum(run, tmax[:, 4 * sp + j])
    rises = np.concatenate(rises)
    assert np.any((rises > 0.5) & (rises < 8.0)) and np.any((rises > 8.0) & (rises < 12.0))
    assert np.any(rises > 12.0)
    ref_o, ref_lse = o.attention_verify(qb, ka, kr, va, vr, B, M, T, Hq, Hkv, 128, P, C, alpha)
    out, lse = lynx.attn_verify(bf16_tensor(qb), upload(ka), upload(kr), upload(va), upload(vr), T, Hkv, P, C,
                                alpha)
    torch.cuda.synchronize()
    bound = lse_bound(qb, ka, kr, B, M, T, Hq, Hkv, P, C, alpha)
    check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_lse, bound,
          "rising")


def test_verify_lse_merges_context_halves(gpu):
    """The LSE returned for two halves of a context merges to the whole (the rule a caller uses to
    add the draft tokens' own keys): O = (e^{l1} O1 + e^{l2} O2) / (e^{l1} + e^{l2})."""
    B, M, Hq, Hkv, T, P, C, alpha = 1, 4, 16, 2, 1024, 256, 64, 255.0
    qb, ka, kr, va, vr = make_case(B, M, Hq, Hkv, T, P, C, alpha, seed=9)
    q = bf16_tensor(qb)
    K, KR, V, VR = upload(ka), upload(kr), upload(va), upload(vr)
    o_all, l_all = lynx.attn_verify(q, K, KR, V, VR, T, Hkv, P, C, alpha)
    h = (T // P) // 2
    o1, l1 = lynx.attn_verify(q, K[:h], KR[:h], V[:h], VR[:h], T // 2, Hkv, P, C, alpha)
    o2, l2 = lynx.attn_verify(q, K[h:], KR[h:], V[h:], VR[h:], T // 2, Hkv, P, C, alpha)
    torch.cuda.synchronize()
    l1, l2, la = (x.double().cpu() for x in (l1, l2, l_all))
    mx = torch.maximum(l1, l2)
    w1, w2 = torch.exp(l1 - mx), torch.exp(l2 - mx)
    merged = (w1[..., None] * o1.double().cpu() + w2[..., None] * o2.double().cpu()) / (w1 + w2)[..., None]
    assert float((mx + torch.log(w1 + w2) - la).abs().max()) <= 1e-5
    assert rel_l2(merged.numpy(), o_all.double().cpu().numpy()) <= 5e-4


def test_verify_full_size_sampled(gpu):
    """16 sequences x 64 draft tokens x 64 query heads / 8 kv heads x 32768 context tokens, P=256, C=64,
    alpha=255, in the launch configuration the benchmark times; the oracle checks two sequences."""
    B, M, Hq, Hkv, T, P, C, alpha = 16, 64, 64, 8, 32768, 256, 64, 255.0
    print("[verify] full size: generating and encoding K/V on the GPU", flush=True)
    kv = torch.empty((B * T, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    codes = []
    for kv_idx in (0, 1):
        for b in range(B):
            synth.make_kv_torch(T, Hkv, 128, seed=0, layer=b, kv_idx=kv_idx, out=kv[b * T:(b + 1) * T])
        codes.extend(lynx.encode(kv, P, C, alpha, residual=True))
    del kv
    ka, kr, va, vr = codes
    q = synth.make_q_torch(B * M, Hq, 128, seed=0).view(B, M, Hq, 128)
    out, lse = lynx.attn_verify(q, ka, kr, va, vr, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    npg = T // P
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    KA, KR, VA, VR = (x.cpu().numpy() for x in (ka, kr, va, vr))
    got, got_lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    for b in (0, 15):
        print(f"[verify] oracle on sequence {b}", flush=True)
        sl = slice(b * npg, (b + 1) * npg)
        ref_o, ref_lse = o.attention_verify(qb[b:b + 1], KA[sl], KR[sl], VA[sl], VR[sl], 1, M, T, Hq, Hkv, 128, P,
                                            C, alpha)
        bound = lse_bound(qb[b:b + 1], KA[sl], KR[sl], 1, M, T, Hq, Hkv, P, C, alpha)
        check(got[b:b + 1], got_lse[b:b + 1], ref_o, ref_lse, bound, f"seq {b}")


@pytest.mark.parametrize("C", [64, 32, 16])
def test_verify_paged_variable_lengths(gpu, C):
    """A shuffled pool of pages behind a block table, with lengths ending inside a tile, on a tile
    edge, inside a page, at one token and at zero (O = 0, LSE = -inf)."""
    B, M, Hq, Hkv, P, maxp, alpha = 6, 3, 16, 2, 256, 4, 255.0
    lens = np.array([1, 63, 64, 300, maxp * P, 0], dtype=np.int32)
    print(f"[verify-paged] C={C} lens={lens.tolist()}", flush=True)
    T = maxp * P
    qb, ka, kr, va, vr = make_case(B, M, Hq, Hkv, T, P, C, alpha, seed=41)
    perm = np.random.default_rng(C + 1).permutation(B * maxp)
    bt = np.argsort(perm)[np.arange(B * maxp).reshape(B, maxp)].astype(np.int32)
    bt[0, 1:] = -1                                   # pages past a sequence's end are not read
    ref_o, ref_l = o.attention_verify_paged(qb, ka[perm], kr[perm], va[perm], vr[perm], bt, lens, Hq, Hkv, 128, P,
                                            C, alpha)
    out, lse = lynx.attn_verify_paged(bf16_tensor(qb), upload(ka[perm]), upload(kr[perm]), upload(va[perm]),
                                      upload(vr[perm]), torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                      Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got_o, got_l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            assert np.all(got_o[b] == 0.0) and np.all(got_l[b] == -np.inf)
            continue
        npg = (n + P - 1) // P
        # the LSE bound of lse_bound, on this sequence's first n tokens
        idx = np.arange(b * maxp, b * maxp + npg)
        K = np.abs(o.decode_full(ka[idx], kr[idx], npg, P, Hkv, 128, C, alpha)[:n])
        q = np.abs(o.bf16_bits_to_f64(qb[b]))
        G = Hq // Hkv
        bound = np.stack([(q[:, h * G:(h + 1) * G].reshape(-1, 128) @ K[:, h, :].T).max(axis=1).reshape(M, G)
                          for h in range(Hkv)], axis=1).reshape(M, Hq) * 2.0 ** -15 / np.sqrt(128)
        check(got_o[b:b + 1], got_l[b:b + 1], ref_o[b:b + 1], ref_l[b:b + 1], bound[None], f"seq {b} len {n}")


def test_verify_group_of_16_long_context(gpu):
    """64 query heads over 4 kv heads (a group of 16), 2 draft tokens, one 32768-token sequence
    encoded on the GPU."""
    B, M, Hq, Hkv, T, P, C, alpha = 1, 2, 64, 4, 32768, 256, 64, 255.0
    kv = [torch.empty((T, Hkv, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for kv_idx in (0, 1):
        synth.make_kv_torch(T, Hkv, 128, seed=8, layer=0, kv_idx=kv_idx, out=kv[kv_idx])
    ka, kr = lynx.encode(kv[0], P, C, alpha)
    va, vr = lynx.encode(kv[1], P, C, alpha)
    q = synth.make_q_torch(B * M, Hq, 128, seed=8).view(B, M, Hq, 128)
    out, lse = lynx.attn_verify(q, ka, kr, va, vr, T, Hkv, P, C, alpha, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qb = q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    KA, KR, VA, VR = (t.cpu().numpy() for t in (ka, kr, va, vr))
    ref_o, ref_lse = o.attention_verify(qb, KA, KR, VA, VR, B, M, T, Hq, Hkv, 128, P, C, alpha)
    bound = lse_bound(qb, KA, KR, B, M, T, Hq, Hkv, P, C, alpha)
    check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_lse, bound,
          "group 16, 32768 tokens")
