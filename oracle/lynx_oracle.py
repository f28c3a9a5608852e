"""Lynx split-stream KV codec and anchor-only decode attention: the CPU oracle.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, float64 statement of
what the GPU path computes.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Sources (cited by page title and section; no other source was used):
  [Review]  "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
            LLM Inference" (technical review of arXiv 2607.01831).
  [Digest]  "Lynx: Progressive Speculative Quantization for accelerating KV
            Transfer in Long-Context Inference" (paper digest), section Method.

Every floating-point step is evaluated in IEEE float64 with numpy, in the order
the pages state it.  Where the pages leave a step open the reading taken is
stated beside the step (readings R-*), and the same list is kept in the
design notes of the repository.

Readings (where the pages are silent, ambiguous or inconsistent):
  R-eps     epsilon is not given on the pages; EPS = 1e-6 in both stages.
  R-meta    metadata is stored as float32 ([Review] Deep Dive, "metadata per
            page in float32"); every later stage uses the stored float32 value,
            so decode(encode) is self-consistent.
  R-sigma   sigma is the per-chunk maximum absolute deviation from the chunk
            mean ([Review] Mechanism 1, Stage 2 pseudocode), which keeps
            X_final inside [-1, 1].
  R-sign    the sign S is taken from X_final (after centring); after Stage 1
            every value is >= 0, so a sign taken there would always be +1.
            S(+-0) = +1.
  R-round   Round(Y) is round-half-to-even; ties have measure zero.
  R-split   Stage 4 as printed adds the +7 bias before the shift, which lets
            the anchor magnitude reach 8 (I = 121..127) and overflow a 4-bit
            two's-complement nibble.  The reading used here moves the +7 to
            the reconstruction point: V_mag = I >> 4, V_recon = 16*V_mag + 7,
            V_res = V_recon - I in [-8, 7], Q_anc = V_mag*S + min(S, 0)
            (Eq. 9 unchanged) in [-8, 7].  Decode recovers I = V_recon - V_res
            exactly, and anchor-only decode is full decode with V_res = 0.
  R-nibble  a 4-bit code q is stored as the nibble q & 0xF (two's complement);
            two codes share a byte, the even element in the low nibble.
  R-layout  within a page, codes are ordered [kv_head][channel block][token][channel
            in block], the head's channels split into blocks of 64 (a head of at
            most 64 channels is one block, i.e. [kv_head][token][head_dim]); a
            page's anchor segment is the anchor nibbles followed by
            gamma_min f32[H], gamma_scale f32[H], mu f32[P/C][H],
            sigma f32[P/C][H] (H = kv_heads*head_dim, channel = h*D + d);
            the residual segment is the residual nibbles alone.
  R-zero    the sign of a zero is not data: a zero gamma_min, gamma_scale or mu is
            stored as +0 whatever the signs of the zeros it comes from.
  R-attn    decode attention is Eq. 1 over the anchor-only reconstruction;
            query head hq uses kv head hq // (Hq/Hkv) (contiguous groups).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6            # R-eps
CODE_MAX = 127        # 2^7 - 1, [Review] Mechanism 1, Stage 3, Eq. 7
SEL_ANCHOR = 1
SEL_RESIDUAL = 2


# ----------------------------------------------------------------------------
# BF16 helpers (exact conversions; no method arithmetic)
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> BF16 bit patterns, one rounding to nearest even.

    Rounds the float64 value directly to the 8-bit significand (no float32
    intermediate), so the result is the correctly rounded BF16 value.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    _, e = np.frexp(flat_x)                     # x = m * 2^e, 0.5 <= |m| < 1
    # keep 8 significant bits (normal range); never finer than the subnormal step 2^-133
    scale_exp = np.minimum(8 - e, 133).astype(np.int64)
    scale = np.ldexp(1.0, scale_exp)
    r = np.rint(flat_x * scale) / scale         # exact scaling by a power of two, RNE
    r32 = r.astype(np.float32)                  # r already has <= 8 significant bits: exact
    flat_o[:] = (r32.view(np.uint32) >> 16).astype(np.uint16)
    return out


# ----------------------------------------------------------------------------
# Stage 1 — per-channel, page-level normalisation
# [Review] Mechanism 1, Stage 1; [Digest] Method, item 1.
# ----------------------------------------------------------------------------
def page_stats(X: np.ndarray):
    """X: [P, H] float64 (exact BF16 values).  Returns (gamma_min, gamma_scale) as float32.

    gamma_min is a BF16 value, so its float32 copy is exact; gamma_scale is the
    float64 range (max - min) rounded once to float32 (R-meta).
    """
    gmin = X.min(axis=0) + 0.0                  # + 0.0: a zero minimum is stored as +0 (R-zero)
    gmax = X.max(axis=0)
    return gmin.astype(np.float32), ((gmax - gmin) + 0.0).astype(np.float32)


def normalize_page(X: np.ndarray, gmin32: np.ndarray, gscale32: np.ndarray) -> np.ndarray:
    """X_n = (X - gamma_min) / (gamma_scale + eps), every channel mapped into [0, 1]."""
    D1 = gscale32.astype(np.float64) + EPS
    return (X - gmin32.astype(np.float64)) / D1


# ----------------------------------------------------------------------------
# Stage 2 — per-channel, chunk-wise outlier isolation
# [Review] Mechanism 1, Stage 2; [Digest] Method, item 2.
# ----------------------------------------------------------------------------
def chunk_view(A: np.ndarray, C: int) -> np.ndarray:
    """[P, H] -> [P/C, C, H]: chunk k holds tokens k*C .. k*C+C-1 of every channel."""
    P, H = A.shape
    assert P % C == 0
    return A.reshape(P // C, C, H)


def chunk_mean(Xn: np.ndarray, C: int):
    """mu per (chunk, channel): the float64 mean, and its float32 stored value (a zero mean of
    negative zeros stored as +0, R-zero)."""
    mu64 = chunk_view(Xn, C).mean(axis=1)
    return mu64, (mu64 + 0.0).astype(np.float32)


def chunk_sigma(Xn: np.ndarray, mu32: np.ndarray, C: int) -> np.ndarray:
    """sigma = max |X_n - mu| over the chunk (R-sigma), taken against the stored mu, stored as float32."""
    dev = np.abs(chunk_view(Xn, C) - mu32.astype(np.float64)[:, None, :])
    return dev.max(axis=1).astype(np.float32)


def isolate_chunks(Xn: np.ndarray, mu32: np.ndarray, sig32: np.ndarray, C: int) -> np.ndarray:
    """X_final = (X_n - mu) / (sigma + eps), in [-1, 1]; returned as [P, H]."""
    D2 = sig32.astype(np.float64) + EPS
    Xf = (chunk_view(Xn, C) - mu32.astype(np.float64)[:, None, :]) / D2[:, None, :]
    return Xf.reshape(Xn.shape)


# ----------------------------------------------------------------------------
# Stage 3 — non-linear alpha-law transform
# [Review] Mechanism 1, Stage 3, Eq. 7 and Eq. 8; [Digest] Method, item 3.
# ----------------------------------------------------------------------------
def alaw_forward(Xf: np.ndarray, alpha: float):
    """Y = ln(1 + a|X_f|) / ln(1 + a) * 127;  I = Round(Y) (R-round);  S = sign (R-sign).

    Returns (Y float64, I int32 in [0, 127], S int32 in {-1, +1}).
    """
    a = float(np.float32(alpha))
    Y = np.log1p(a * np.abs(Xf)) / np.log1p(a) * CODE_MAX
    I = np.clip(np.rint(Y), 0, CODE_MAX).astype(np.int32)
    S = np.where(Xf < 0, -1, 1).astype(np.int32)
    return Y, I, S


def alaw_inverse(I: np.ndarray, alpha: float) -> np.ndarray:
    """|x_hat| = ((1 + a)^(I/127) - 1) / a  (Eq. 8, normalised so that I=0 -> 0 and I=127 -> 1,
    as in the worked example, Eq. 14 and Eq. 15)."""
    a = float(np.float32(alpha))
    return np.expm1(np.asarray(I, dtype=np.float64) / CODE_MAX * np.log1p(a)) / a


# ----------------------------------------------------------------------------
# Stage 4 — split-stream construction
# [Review] Mechanism 1, Stage 4 and Eq. 9; [Digest] Method, item 4.
# ----------------------------------------------------------------------------
def split_streams(I: np.ndarray, S: np.ndarray):
    """Reading R-split.  Returns (Q_anc, Q_res), both int32 in [-8, 7]."""
    I = np.asarray(I, dtype=np.int32)
    S = np.asarray(S, dtype=np.int32)
    V_mag = I >> 4
    V_recon = (V_mag << 4) + 7
    V_res = V_recon - I
    Q_anc = V_mag * S + np.minimum(S, 0)        # Eq. 9
    return Q_anc.astype(np.int32), V_res.astype(np.int32)


def anchor_sign_mag(Q_anc: np.ndarray):
    """Invert Eq. 9: S = -1 iff Q_anc < 0; V_mag = Q_anc (S=+1) or -Q_anc - 1 (S=-1)."""
    Q = np.asarray(Q_anc, dtype=np.int32)
    S = np.where(Q < 0, -1, 1).astype(np.int32)
    V_mag = np.where(Q < 0, -Q - 1, Q).astype(np.int32)
    return S, V_mag


def code_anchor_only(Q_anc: np.ndarray):
    """Anchor-only reconstruction of the 7-bit code: I_a = 16*V_mag + 7 (R-split, V_res taken as 0)."""
    S, V_mag = anchor_sign_mag(Q_anc)
    return S, 16 * V_mag + 7


def code_full(Q_anc: np.ndarray, Q_res: np.ndarray):
    """Anchor + Residual: I = V_recon - V_res, the exact 7-bit code ([Review] worked example, Eq. 15)."""
    S, V_mag = anchor_sign_mag(Q_anc)
    return S, 16 * V_mag + 7 - np.asarray(Q_res, dtype=np.int32)


def denormalize(S, mag, mu32, sig32, gmin32, gscale32, C: int) -> np.ndarray:
    """Undo Stage 2 then Stage 1: X_hat = ((S*|x_hat|)*(sigma+eps) + mu)*(gamma_scale+eps) + gamma_min.

    S, mag: [P, H]; mu32, sig32: [P/C, H]; gmin32, gscale32: [H].  Returns [P, H] float64.
    """
    P, H = np.shape(mag)
    xf = (np.asarray(S, dtype=np.float64) * np.asarray(mag, dtype=np.float64)).reshape(P // C, C, H)
    D2 = sig32.astype(np.float64)[:, None, :] + EPS
    xn = xf * D2 + mu32.astype(np.float64)[:, None, :]
    D1 = gscale32.astype(np.float64) + EPS
    return (xn * D1 + gmin32.astype(np.float64)).reshape(P, H)


# ----------------------------------------------------------------------------
# One page, end to end (Algorithm 1 of [Review] Mechanism 1)
# ----------------------------------------------------------------------------
def encode_page(X: np.ndarray, C: int, alpha: float) -> dict:
    """X: [P, H] float64 (exact BF16 values).  Runs Stages 1-4 and returns every intermediate."""
    gmin, gscale = page_stats(X)
    Xn = normalize_page(X, gmin, gscale)
    mu64, mu = chunk_mean(Xn, C)
    sig = chunk_sigma(Xn, mu, C)
    Xf = isolate_chunks(Xn, mu, sig, C)
    Y, I, S = alaw_forward(Xf, alpha)
    Q_anc, Q_res = split_streams(I, S)
    return dict(gmin=gmin, gscale=gscale, mu=mu, mu64=mu64, sigma=sig,
                Xn=Xn, Xf=Xf, Y=Y, I=I, S=S, Q_anc=Q_anc, Q_res=Q_res)


def codes_given_metadata(X: np.ndarray, gmin32, gscale32, mu32, sig32, C: int, alpha: float) -> dict:
    """Stages 2-4 of one page run against given (stored) metadata instead of recomputed metadata."""
    Xn = normalize_page(X, gmin32, gscale32)
    Xf = isolate_chunks(Xn, mu32, sig32, C)
    Y, I, S = alaw_forward(Xf, alpha)
    Q_anc, Q_res = split_streams(I, S)
    return dict(Xf=Xf, Y=Y, I=I, S=S, Q_anc=Q_anc, Q_res=Q_res)


def decode_page_anchor(Q_anc, mu32, sig32, gmin32, gscale32, C: int, alpha: float) -> np.ndarray:
    """Q_approx = dequant(Q_anc, gamma, mu, sigma)  ([Review] Mechanism 2, decode-side anchor phase)."""
    S, I_a = code_anchor_only(Q_anc)
    return denormalize(S, alaw_inverse(I_a, alpha), mu32, sig32, gmin32, gscale32, C)


def decode_page_full(Q_anc, Q_res, mu32, sig32, gmin32, gscale32, C: int, alpha: float) -> np.ndarray:
    """Q_full = dequant(Q_anc + Q_res)  ([Review] Mechanism 2, decode-side residual phase)."""
    S, I = code_full(Q_anc, Q_res)
    return denormalize(S, alaw_inverse(I, alpha), mu32, sig32, gmin32, gscale32, C)


# ----------------------------------------------------------------------------
# Stream layout (R-nibble, R-layout; [Review] Implementation Notes: two 4-bit
# values per uint8; Mechanism 2: anchor codes and metadata contiguous)
# ----------------------------------------------------------------------------
def metadata_scalars(P: int, H: int, C: int) -> int:
    """H * (2 + 2P/C) float32 scalars per page ([Review] Deep Dive, metadata count)."""
    return H * (2 + 2 * (P // C))


def segment_bytes(P: int, Hkv: int, D: int, C: int):
    """(anchor segment bytes, residual segment bytes) for one page."""
    H = Hkv * D
    codes = P * H // 2
    return codes + 4 * metadata_scalars(P, H, C), codes


CODE_BLOCK = 64       # channels of one code block (R-layout)


def _code_blocks(D: int) -> int:
    """Channel blocks per kv head: 1 for D <= 64, else D / 64 (R-layout)."""
    if D <= CODE_BLOCK:
        return 1
    assert D % CODE_BLOCK == 0, "head_dim above 64 must be a multiple of 64"
    return D // CODE_BLOCK


def pack_nibbles(Q: np.ndarray, Hkv: int, D: int) -> np.ndarray:
    """Q: [P, H] codes in [-8, 7] -> P*H/2 bytes in [kv_head][channel block][token][channel] order
    (R-layout), even element in the low nibble (R-nibble)."""
    P, H = Q.shape
    nb = _code_blocks(D)
    order = np.asarray(Q, dtype=np.int32).reshape(P, Hkv, nb, D // nb).transpose(1, 2, 0, 3).reshape(-1)
    nib = (order & 0xF).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray, P: int, Hkv: int, D: int) -> np.ndarray:
    """Inverse of pack_nibbles: bytes -> [P, H] signed codes in [-8, 7]."""
    b = np.asarray(b, dtype=np.uint8)
    nb = _code_blocks(D)
    nib = np.empty(b.size * 2, dtype=np.int32)
    nib[0::2] = b & 0xF
    nib[1::2] = b >> 4
    q = np.where(nib >= 8, nib - 16, nib)
    return q.reshape(Hkv, nb, P, D // nb).transpose(2, 0, 1, 3).reshape(P, Hkv * D)


def build_anchor_segment(enc: dict, Hkv: int, D: int) -> np.ndarray:
    meta = np.concatenate([enc["gmin"].reshape(-1), enc["gscale"].reshape(-1),
                           enc["mu"].reshape(-1), enc["sigma"].reshape(-1)]).astype("<f4")
    return np.concatenate([pack_nibbles(enc["Q_anc"], Hkv, D), meta.view(np.uint8)])


def parse_anchor_segment(seg: np.ndarray, P: int, Hkv: int, D: int, C: int) -> dict:
    H = Hkv * D
    seg = np.asarray(seg, dtype=np.uint8)
    codes = P * H // 2
    meta = seg[codes:codes + 4 * metadata_scalars(P, H, C)].view("<f4")
    nck = P // C
    return dict(Q_anc=unpack_nibbles(seg[:codes], P, Hkv, D),
                gmin=meta[:H].copy(), gscale=meta[H:2 * H].copy(),
                mu=meta[2 * H:2 * H + nck * H].reshape(nck, H).copy(),
                sigma=meta[2 * H + nck * H:].reshape(nck, H).copy())


# ----------------------------------------------------------------------------
# Whole tensors of pages (what the library entry points take and return)
# ----------------------------------------------------------------------------
def encode(kv_bits: np.ndarray, P: int, C: int, alpha: float):
    """kv_bits: [n_pages*P, Hkv, D] uint16 BF16 patterns.

    Returns (anchor bytes [n_pages, anchor_seg], residual bytes [n_pages, residual_seg], list of per-page dicts).
    """
    T, Hkv, D = kv_bits.shape
    assert T % P == 0
    n_pages = T // P
    a_sz, r_sz = segment_bytes(P, Hkv, D, C)
    anchor = np.empty((n_pages, a_sz), dtype=np.uint8)
    residual = np.empty((n_pages, r_sz), dtype=np.uint8)
    pages = []
    for p in range(n_pages):
        X = bf16_bits_to_f64(kv_bits[p * P:(p + 1) * P]).reshape(P, Hkv * D)
        enc = encode_page(X, C, alpha)
        anchor[p] = build_anchor_segment(enc, Hkv, D)
        residual[p] = pack_nibbles(enc["Q_res"], Hkv, D)
        pages.append(enc)
    return anchor, residual, pages


def decode_anchor(anchor: np.ndarray, n_pages: int, P: int, Hkv: int, D: int, C: int, alpha: float) -> np.ndarray:
    """Anchor segments -> [n_pages*P, Hkv, D] float64."""
    a_sz, _ = segment_bytes(P, Hkv, D, C)
    anchor = np.asarray(anchor, dtype=np.uint8).reshape(n_pages, a_sz)
    out = np.empty((n_pages * P, Hkv, D), dtype=np.float64)
    for p in range(n_pages):
        m = parse_anchor_segment(anchor[p], P, Hkv, D, C)
        out[p * P:(p + 1) * P] = decode_page_anchor(m["Q_anc"], m["mu"], m["sigma"], m["gmin"],
                                                    m["gscale"], C, alpha).reshape(P, Hkv, D)
    return out


def decode_full(anchor: np.ndarray, residual: np.ndarray, n_pages: int, P: int, Hkv: int, D: int,
                C: int, alpha: float) -> np.ndarray:
    """Anchor + residual segments -> [n_pages*P, Hkv, D] float64."""
    a_sz, r_sz = segment_bytes(P, Hkv, D, C)
    anchor = np.asarray(anchor, dtype=np.uint8).reshape(n_pages, a_sz)
    residual = np.asarray(residual, dtype=np.uint8).reshape(n_pages, r_sz)
    out = np.empty((n_pages * P, Hkv, D), dtype=np.float64)
    for p in range(n_pages):
        m = parse_anchor_segment(anchor[p], P, Hkv, D, C)
        Q_res = unpack_nibbles(residual[p], P, Hkv, D)
        out[p * P:(p + 1) * P] = decode_page_full(m["Q_anc"], Q_res, m["mu"], m["sigma"], m["gmin"],
                                                  m["gscale"], C, alpha).reshape(P, Hkv, D)
    return out


# ----------------------------------------------------------------------------
# Decode attention, Eq. 1 of [Review] Prerequisites §1, over the anchor-only
# reconstruction (the draft path of [Review] Mechanism 2 / 3).
# ----------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float | None = None) -> np.ndarray:
    """q: [B, Hq, D]; K, V: [B, T, Hkv, D] (float64).  O = softmax(q K^T * scale) V, per head (R-attn)."""
    B, Hq, D = q.shape
    _, T, Hkv, _ = K.shape
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if sm_scale is None else float(sm_scale)
    O = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            qg = np.asarray(q[b, h * G:(h + 1) * G], dtype=np.float64)
            s = (qg @ K[b, :, h, :].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            O[b, h * G:(h + 1) * G] = p @ V[b, :, h, :]
    return O


def attention_anchor(q_bits: np.ndarray, k_anchor: np.ndarray, v_anchor: np.ndarray, batch: int, ctx: int,
                     Hq: int, Hkv: int, D: int, P: int, C: int, alpha: float,
                     sm_scale: float | None = None) -> np.ndarray:
    """q_bits: [B, Hq, D] BF16 patterns; k_anchor/v_anchor: B*ctx/P anchor segments, sequence-major.

    Returns O [B, Hq, D] float64 = Eq. 1 over the anchor-only decode of K and V.
    """
    n_pages = ctx // P
    q = bf16_bits_to_f64(q_bits)
    a_sz, _ = segment_bytes(P, Hkv, D, C)
    k_anchor = np.asarray(k_anchor, dtype=np.uint8).reshape(batch, n_pages * a_sz)
    v_anchor = np.asarray(v_anchor, dtype=np.uint8).reshape(batch, n_pages * a_sz)
    O = np.empty((batch, Hq, D), dtype=np.float64)
    for b in range(batch):
        Kh = decode_anchor(k_anchor[b], n_pages, P, Hkv, D, C, alpha)[None]
        Vh = decode_anchor(v_anchor[b], n_pages, P, Hkv, D, C, alpha)[None]
        O[b] = attention(q[b:b + 1], Kh, Vh, sm_scale)[0]
    return O


def attention_anchor_paged(q_bits: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
                           seq_lens: np.ndarray, Hq: int, Hkv: int, D: int, P: int, C: int, alpha: float,
                           sm_scale: float | None = None) -> np.ndarray:
    """Eq. 1 over a paged anchor cache with per-sequence lengths.

    q_bits [B, Hq, D]; k_pool / v_pool: pool of anchor segments [n_pool, anchor_seg]; block_table
    [B, max_pages] (entry (b, p) = pool segment of page p of sequence b); seq_lens [B].  Sequence b's
    context is the first seq_lens[b] tokens of its pages in order; an empty context gives O = 0.
    """
    q = bf16_bits_to_f64(q_bits)
    B = q.shape[0]
    O = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        pages = [int(x) for x in block_table[b, :(n + P - 1) // P]]
        Kh = decode_anchor(np.asarray(k_pool)[pages], len(pages), P, Hkv, D, C, alpha)[:n][None]
        Vh = decode_anchor(np.asarray(v_pool)[pages], len(pages), P, Hkv, D, C, alpha)[:n][None]
        O[b] = attention(q[b:b + 1], Kh, Vh, sm_scale)[0]
    return O


def attention_lse(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float | None = None):
    """q: [R, Hq, D] (R query tokens); K, V: [T, Hkv, D] (float64), shared by the R queries.

    Returns (O [R, Hq, D], lse [R, Hq]): Eq. 1 per query token and head (R-attn grouping), and the
    natural-log log-sum-exp of the scaled scores, log(sum_t exp(s_t)) with s_t = scale * q . k_t.
    """
    R, Hq, D = q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if sm_scale is None else float(sm_scale)
    O = np.empty((R, Hq, D), dtype=np.float64)
    lse = np.empty((R, Hq), dtype=np.float64)
    for h in range(Hkv):
        qg = np.asarray(q[:, h * G:(h + 1) * G, :], dtype=np.float64).reshape(R * G, D)
        s = (qg @ K[:, h, :].T) * scale
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        tot = e.sum(axis=1, keepdims=True)
        O[:, h * G:(h + 1) * G, :] = ((e / tot) @ V[:, h, :]).reshape(R, G, D)
        lse[:, h * G:(h + 1) * G] = (m + np.log(tot)).reshape(R, G)
    return O, lse


def attention_verify(q_bits: np.ndarray, k_anchor: np.ndarray, k_residual: np.ndarray, v_anchor: np.ndarray,
                     v_residual: np.ndarray, batch: int, n_query: int, ctx: int, Hq: int, Hkv: int, D: int,
                     P: int, C: int, alpha: float, sm_scale: float | None = None):
    """The verification pass ([Review] Mechanism 3, single parallel verification pass, with Eq. 1): each of
    the n_query draft tokens of sequence b attends to the ctx context tokens whose K and V are the full
    decode, Q_full = dequant(Q_anc + Q_res) (Mechanism 2, residual phase).

    q_bits: [B, n_query, Hq, D] BF16 patterns; *_anchor / *_residual: B*ctx/P segments, sequence-major.
    Returns (O [B, n_query, Hq, D], lse [B, n_query, Hq]) in float64; lse is the natural-log log-sum-exp
    of each query's scaled scores over the context (what a caller needs to merge this result with the
    draft tokens' attention over themselves, which is not in the compressed cache).
    """
    n_pages = ctx // P
    q = bf16_bits_to_f64(q_bits)
    a_sz, r_sz = segment_bytes(P, Hkv, D, C)
    ka = np.asarray(k_anchor, dtype=np.uint8).reshape(batch, n_pages * a_sz)
    kr = np.asarray(k_residual, dtype=np.uint8).reshape(batch, n_pages * r_sz)
    va = np.asarray(v_anchor, dtype=np.uint8).reshape(batch, n_pages * a_sz)
    vr = np.asarray(v_residual, dtype=np.uint8).reshape(batch, n_pages * r_sz)
    O = np.empty((batch, n_query, Hq, D), dtype=np.float64)
    lse = np.empty((batch, n_query, Hq), dtype=np.float64)
    for b in range(batch):
        Kh = decode_full(ka[b], kr[b], n_pages, P, Hkv, D, C, alpha)
        Vh = decode_full(va[b], vr[b], n_pages, P, Hkv, D, C, alpha)
        O[b], lse[b] = attention_lse(q[b], Kh, Vh, sm_scale)
    return O, lse


def attention_verify_paged(q_bits: np.ndarray, ka_pool: np.ndarray, kr_pool: np.ndarray, va_pool: np.ndarray,
                           vr_pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray, Hq: int, Hkv: int,
                           D: int, P: int, C: int, alpha: float, sm_scale: float | None = None):
    """The verification pass over a paged cache with per-sequence lengths.

    q_bits [B, M, Hq, D]; pools of anchor / residual segments ([n_pool, seg], pool segment s of both
    streams is one page); block_table [B, max_pages]; seq_lens [B].  Sequence b's context is the
    first seq_lens[b] tokens of its pages in order.  Returns (O, lse); an empty context gives O = 0
    and lse = -inf.
    """
    q = bf16_bits_to_f64(q_bits)
    B, M = q.shape[:2]
    O = np.zeros((B, M, Hq, D), dtype=np.float64)
    lse = np.full((B, M, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        pages = [int(x) for x in block_table[b, :(n + P - 1) // P]]
        Kh = decode_full(np.asarray(ka_pool)[pages], np.asarray(kr_pool)[pages], len(pages), P, Hkv, D, C, alpha)
        Vh = decode_full(np.asarray(va_pool)[pages], np.asarray(vr_pool)[pages], len(pages), P, Hkv, D, C, alpha)
        O[b], lse[b] = attention_lse(q[b], Kh[:n], Vh[:n], sm_scale)
    return O, lse
