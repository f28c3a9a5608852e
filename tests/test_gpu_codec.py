"""GPU parity of the codec (encode, anchor-only decode, full decode) against the oracle.

Every page the oracle checks is compared element by element under the contract
written in tests/parity.py.  Cases span several 256-token tiles, ragged tails,
every supported chunk size, the three alpha values of the sweep, and the
degenerate inputs the method has (constant channels and chunks, signed zeros,
extreme magnitudes).
"""
import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth
from oracle import lynx_oracle as o
from tests import parity

pytestmark = pytest.mark.gpu


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run_codec(bits: np.ndarray, P: int, C: int, alpha: float, pages=None, label="", bf16_share=parity.CODE_FLIP_FRAC):
    """Encode + both decoders on the GPU; oracle comparison on `pages` (default: all)."""
    T, Hkv, D = bits.shape
    n_pages = T // P
    print(f"[codec] {label} T={T} Hkv={Hkv} P={P} C={C} alpha={alpha}", flush=True)
    kv = to_dev(bits)
    anc, res = lynx.encode(kv, P, C, alpha)
    outs = {
        "anc32": lynx.decode_anchor(anc, n_pages, P, Hkv, D, C, alpha, out_dtype=torch.float32),
        "full32": lynx.decode_full(anc, res, n_pages, P, Hkv, D, C, alpha, out_dtype=torch.float32),
        "anc16": lynx.decode_anchor(anc, n_pages, P, Hkv, D, C, alpha),
        "full16": lynx.decode_full(anc, res, n_pages, P, Hkv, D, C, alpha),
    }
    torch.cuda.synchronize()
    A, R = anc.cpu().numpy(), res.cpu().numpy()
    host = {k: v.cpu() for k, v in outs.items()}
    H = Hkv * D
    rep = {}
    for p in (range(n_pages) if pages is None else pages):
        X = o.bf16_bits_to_f64(bits[p * P:(p + 1) * P]).reshape(P, H)
        enc = o.encode_page(X, C, alpha)
        got = o.parse_anchor_segment(A[p], P, Hkv, D, C)
        q_res = o.unpack_nibbles(R[p], P, Hkv, D)
        parity.check_metadata(got, enc, X, C, rep)
        parity.check_codes(got, q_res, X, C, alpha, rep)
        args = (got["mu"], got["sigma"], got["gmin"], got["gscale"], C, alpha)
        ref_full = o.decode_page_full(got["Q_anc"], q_res, *args)
        ref_anc = o.decode_page_anchor(got["Q_anc"], *args)
        sl = slice(p * P, (p + 1) * P)
        parity.check_decode_f32(host["full32"][sl].numpy().reshape(P, H), ref_full, got["gscale"], rep)
        parity.check_decode_f32(host["anc32"][sl].numpy().reshape(P, H), ref_anc, got["gscale"], rep)
        parity.check_decode_bf16(host["full16"][sl].view(torch.int16).numpy().view(np.uint16).reshape(P, H),
                                 ref_full, parity.decode_slack(got, ref_full, C), rep)
        parity.check_decode_bf16(host["anc16"][sl].view(torch.int16).numpy().view(np.uint16).reshape(P, H),
                                 ref_anc, parity.decode_slack(got, ref_anc, C), rep)
    parity.finish_codes(rep)
    parity.finish_bf16(rep, bf16_share)
    print(f"[codec] {label} report {rep}", flush=True)
    return anc, res, rep


def test_single_page_4096_tokens_k_and_v(gpu):
    """One 4096-token page of K and of V, 8 kv heads x 128, C = 64, alpha = 255, seed 0."""
    for kv_idx in (0, 1):
        bits = synth.make_kv_np(4096, 8, 128, seed=0, layer=0, kv_idx=kv_idx)
        run_codec(bits, 4096, 64, 255.0, label=f"page4096 kv{kv_idx}")


@pytest.mark.parametrize("P,C,alpha,Hkv,n_pages", [
    (256, 64, 255.0, 2, 3),
    (256, 8, 15.0, 1, 2),
    (256, 16, 63.0, 1, 2),
    (256, 32, 255.0, 2, 1),
    (256, 128, 63.0, 1, 2),
    (256, 256, 15.0, 1, 2),
    (320, 64, 255.0, 1, 2),     # 256-token tile plus a 64-token ragged tile
    (24, 8, 255.0, 1, 3),       # a page shorter than one tile
    (512, 256, 255.0, 1, 1),    # chunk spanning all four waves, two tiles
    (768, 128, 63.0, 1, 1),
    (64, 64, 100.0, 4, 2),
    (264, 8, 255.0, 1, 2),      # long page: a full tile plus an 8-token tile, the smallest chunk
    (1024, 256, 63.0, 2, 1),    # four tiles of one 256-token chunk each
    (2048, 32, 15.0, 1, 2),     # eight tiles, two pages
    (256, 64, 1.0, 2, 2),       # alpha 1: the compander close to linear
    (256, 32, 4096.0, 1, 2),    # a very large alpha
])
def test_codec_shapes(gpu, P, C, alpha, Hkv, n_pages):
    bits = synth.make_kv_np(P * n_pages, Hkv, 128, seed=P + C, layer=Hkv)
    run_codec(bits, P, C, alpha, label=f"shape P{P} C{C}")


@pytest.mark.parametrize("P", [256, 512])
def test_degenerate_pages(gpu, P):
    """Constant channels (at zero, negative, with -0.0), a constant chunk inside a live
    channel, huge and tiny magnitudes, and an all-constant page; P = 512 takes the
    two-tile path, whose page extremes are reduced across workgroups."""
    C, Hkv, D = 32, 1, 128
    rng = np.random.default_rng(7)
    X = rng.laplace(0, 0.5, size=(2 * P, Hkv, D)).astype(np.float32)
    X[:, 0, 0] = 0.0
    X[:, 0, 1] = -3.5
    X[::2, 0, 2] = -0.0
    X[1::2, 0, 2] = 0.0
    X[64:96, 0, 3] = 1.25                          # one constant chunk in a live channel
    X[:, 0, 4] *= 1e30                             # huge values
    X[:, 0, 5] *= 1e-30                            # tiny values (normal BF16)
    X[:, 0, 6] = np.where(np.arange(2 * P) % 2 == 0, 1e-38, -1e-38)   # near the subnormal range
    X[P:, 0, 7:] = 2.0                             # second page: constant except channels 0..6
    X[:, 0, 8] = rng.choice([-1.0, 1.0], size=2 * P) * 2.0 ** rng.integers(-20, 20, size=2 * P)
    X[:, 0, 9] = np.abs(X[:, 0, 9])                # minimum zero ...
    X[:32, 0, 9] = -0.0                            # ... and a chunk of negative zeros: mu = 0 stored as +0
    bits = o.f64_to_bf16_bits(X.astype(np.float64))
    run_codec(bits, P, C, 255.0, label=f"degenerate P{P}", bf16_share=None)


def test_zero_pages_is_a_noop(gpu):
    kv = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    sentinel = torch.full((1, 16), 0xAB, dtype=torch.uint8, device="cuda")
    st = lynx.lib().lynx_encode(lynx._ptr(kv), 0, 256, 8, 128, 64, 255.0, 3, lynx._ptr(sentinel),
                                lynx._ptr(sentinel), None)
    torch.cuda.synchronize()
    assert st == lynx.LYNX_OK and bool((sentinel == 0xAB).all())


def test_anchor_only_encode_matches_full_encode(gpu):
    """sel = ANCHOR writes the same anchor segment as sel = ANCHOR | RESIDUAL."""
    bits = synth.make_kv_np(512, 2, 128, seed=3)
    kv = to_dev(bits)
    a1, r1 = lynx.encode(kv, 256, 64, 255.0)
    a2, r2 = lynx.encode(kv, 256, 64, 255.0, residual=False)
    torch.cuda.synchronize()
    assert r2 is None and torch.equal(a1, a2)


def test_calls_on_two_streams_match_one_stream(gpu):
    """The library keeps no state between calls: per-tensor encodes and decodes alternating
    over two streams (running concurrently) give the bytes of the same calls on one stream."""
    P, C, alpha, Hkv, D = 256, 64, 255.0, 4, 128
    n_t, tokens = 6, 1024
    kv = torch.cat([to_dev(synth.make_kv_np(tokens, Hkv, D, seed=9, layer=t)) for t in range(n_t)])
    ppt = tokens // P
    a_sz, r_sz = lynx.stream_sizes(P, Hkv, D, C)

    def run(streams):
        anc = torch.zeros((n_t * ppt, a_sz), dtype=torch.uint8, device="cuda")
        res = torch.zeros((n_t * ppt, r_sz), dtype=torch.uint8, device="cuda")
        outs = [torch.zeros((tokens, Hkv, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_t)]
        main = torch.cuda.current_stream()
        for st in streams:
            st.wait_stream(main)
        for t in range(n_t):
            st = streams[t % len(streams)]
            sl = slice(t * ppt, (t + 1) * ppt)
            lynx.encode(kv[t * tokens:(t + 1) * tokens], P, C, alpha, anchor_out=anc[sl], residual_out=res[sl],
                        stream=st)
            lynx.decode_full(anc[sl], res[sl], ppt, P, Hkv, D, C, alpha, out=outs[t], stream=st)
        for st in streams:
            main.wait_stream(st)
        torch.cuda.synchronize()
        return anc, res, torch.stack(outs)

    one = run([torch.cuda.current_stream()])
    two = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for x, y in zip(one, two):
        assert torch.equal(x, y)


def test_binding_refuses_undersized_or_mistyped_device_buffers(gpu):
    """A buffer the kernels would overrun, or read in the wrong format, is refused on the host."""
    P, C, alpha, Hkv, D = 256, 64, 255.0, 2, 128
    kv = to_dev(synth.make_kv_np(2 * P, Hkv, D, seed=4))
    a_sz, r_sz = lynx.stream_sizes(P, Hkv, D, C)
    small = torch.empty((1, a_sz), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="anchor_out"):
        lynx.encode(kv, P, C, alpha, anchor_out=small)
    anc, res = lynx.encode(kv, P, C, alpha)
    with pytest.raises(ValueError, match="residual"):
        lynx.decode_full(anc, res[:1], 2, P, Hkv, D, C, alpha)
    with pytest.raises(ValueError, match="dtype"):
        lynx.decode_anchor(anc, 2, P, Hkv, D, C, alpha, out=torch.empty((2 * P, Hkv, D), dtype=torch.float16,
                                                                        device="cuda"))
    with pytest.raises(ValueError, match="out"):
        lynx.decode_anchor(anc, 2, P, Hkv, D, C, alpha, out=torch.empty((P, Hkv, D), dtype=torch.bfloat16,
                                                                        device="cuda"))
    q32 = torch.zeros((1, 4, D), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="q"):
        lynx.attn_anchor(q32, anc, anc, 2 * P, Hkv, P, C, alpha)
    q = q32.to(torch.bfloat16)
    with pytest.raises(ValueError, match="k_anchor"):
        lynx.attn_anchor(q, anc[:1], anc, 2 * P, Hkv, P, C, alpha)
    torch.cuda.synchronize()
