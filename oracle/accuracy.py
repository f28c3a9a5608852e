"""Accuracy of the Lynx codec on synthetic KV: vNMSE of attention outputs (CPU, float64).

TEST INFRASTRUCTURE ONLY, under the same rule as `lynx_oracle`: only the test
suite, the smoke check, the benchmark's CPU leg and the scripts under
`tests/golden/` use it.  It builds on the oracle's codec and attention and adds
the comparison quantisers and the error measure.

Sources (cited by page title and section):
  [Review]  "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
            LLM Inference" (technical review of arXiv 2607.01831):
            Prerequisites §4, Eq. 4 (linear quantisation) and Eq. 5 (effective
            bins); Setup (the Lynx, Lynx-INT4 and Lynx-INT8 configurations and
            the INT4 / INT8 baselines); the vNMSE table of attention outputs;
            the reviewer's suggested ablations (bit splits 3+5 .. 6+2, alpha,
            C and P).

Readings (the pages name these quantities without defining them):
  A-vnmse   vNMSE = sum ||O_q - O||^2 / sum ||O||^2 over every query token and
            query head, O the attention output over the exact BF16 KV and O_q
            the output over the reconstructed KV (same queries).
  A-linear  Eq. 4 is applied per group of one token's head_dim channels of one
            kv head (asymmetric, per-token): S = (max - min) / (2^B - 1),
            zero point Z = round(-min / S), Q = clip(round(x / S + Z), 0,
            2^B - 1), x_hat = (Q - Z) S.  A constant group (S = 0) is exact.
            This is the granularity at which Eq. 5's outlier argument bites:
            an outlier channel sets S for the whole token.
  A-int4    "Lynx-INT4" (quantise only, no split stream) is the anchor stream
            alone: 4-bit alpha-law codes with Lynx's page / chunk metadata,
            decoded by the anchor-only decoder.
  A-int8    "Lynx-INT8" (standard INT8 split into anchor + residual) is the
            A-linear INT8 code split into its high nibble (anchor) and low
            nibble (residual).  Its full decode is INT8; its anchor-only
            decode takes the low nibble at its mid-range: Q ~ 16 hi + 7.5.
  A-split   A bit split a + (8 - a) keeps the sign and the top a - 1 bits of
            the 7-bit code I in the anchor: V_mag = I >> (8 - a), anchor-only
            code I_a = V_mag 2^(8-a) + 2^(7-a) - 1, residual I_a - I in
            [-2^(7-a), 2^(7-a) - 1] (8 - a bits).  a = 4 is reading R-split of
            the codec.  The full decode recovers I whatever the split.
"""
from __future__ import annotations

import numpy as np

from . import lynx_oracle as o


def vnmse(O_q: np.ndarray, O_ref: np.ndarray) -> float:
    """A-vnmse."""
    O_q = np.asarray(O_q, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    return float(np.sum((O_q - O_ref) ** 2) / np.sum(O_ref ** 2))


def linear_codes(x: np.ndarray, bits: int):
    """Eq. 4 per group along the last axis (A-linear).  Returns (Q int, S, Z) with S and Z
    broadcastable against x."""
    x = np.asarray(x, dtype=np.float64)
    levels = 2 ** bits - 1
    xmin = x.min(axis=-1, keepdims=True)
    xmax = x.max(axis=-1, keepdims=True)
    S = (xmax - xmin) / levels
    safe = np.where(S > 0, S, 1.0)
    Z = np.where(S > 0, np.rint(-xmin / safe), 0.0)
    Q = np.where(S > 0, np.clip(np.rint(x / safe + Z), 0, levels), 0.0)
    return Q.astype(np.int64), S, Z


def linear_dequant(Q: np.ndarray, S: np.ndarray, Z: np.ndarray, xmin: np.ndarray | None = None) -> np.ndarray:
    """x_hat = (Q - Z) S; a constant group (S = 0) returns its value, passed as xmin."""
    xh = (np.asarray(Q, dtype=np.float64) - Z) * S
    if xmin is not None:
        xh = np.where(S > 0, xh, xmin)
    return xh


def linear_roundtrip(x: np.ndarray, bits: int) -> np.ndarray:
    """Quantise and dequantise with Eq. 4 (A-linear)."""
    x = np.asarray(x, dtype=np.float64)
    Q, S, Z = linear_codes(x, bits)
    return linear_dequant(Q, S, Z, x.min(axis=-1, keepdims=True))


def int8_split_anchor(x: np.ndarray) -> np.ndarray:
    """Lynx-INT8 anchor-only reconstruction (A-int8): the high nibble of the INT8 code, the low
    nibble taken at its mid-range."""
    x = np.asarray(x, dtype=np.float64)
    Q, S, Z = linear_codes(x, 8)
    hi = Q >> 4
    return linear_dequant(16.0 * hi + 7.5, S, Z, x.min(axis=-1, keepdims=True))


def split_anchor_code(I: np.ndarray, a: int) -> np.ndarray:
    """A-split: the anchor-only 7-bit code of an a + (8 - a) split (a = 4 gives 16 V_mag + 7)."""
    if not 2 <= a <= 8:
        raise ValueError("the anchor keeps the sign and 1..7 magnitude bits")
    I = np.asarray(I, dtype=np.int64)
    r = 8 - a
    return ((I >> r) << r) + (2 ** (r - 1) - 1 if r > 0 else 0)


def lynx_pages(kv_bits: np.ndarray, P: int, C: int, alpha: float):
    """Run the oracle encoder; returns (per-page dicts, Hkv, D)."""
    _, _, pages = o.encode(kv_bits, P, C, alpha)
    return pages, kv_bits.shape[1], kv_bits.shape[2]


def lynx_reconstruct(pages, P: int, Hkv: int, D: int, C: int, alpha: float, anchor_bits: int | None) -> np.ndarray:
    """[n_pages*P, Hkv, D] reconstruction from the oracle's page codes: the full decode
    (anchor_bits None) or the anchor-only decode of an anchor_bits split (A-split)."""
    out = []
    for enc in pages:
        if anchor_bits is None:
            S, I = enc["S"], enc["I"]
        else:
            S, I = enc["S"], split_anchor_code(enc["I"], anchor_bits)
        x = o.denormalize(S, o.alaw_inverse(I, alpha), enc["mu"], enc["sigma"], enc["gmin"], enc["gscale"], C)
        out.append(x.reshape(P, Hkv, D))
    return np.concatenate(out)


def attention_outputs(q_bits: np.ndarray, K: np.ndarray, V: np.ndarray, T: int) -> np.ndarray:
    """q_bits [B, M, Hq, D]; K, V [B*T, Hkv, D] float64.  Eq. 1 for every query: [B, M, Hq, D]."""
    B = q_bits.shape[0]
    q = o.bf16_bits_to_f64(q_bits)
    return np.stack([o.attention_lse(q[b], K[b * T:(b + 1) * T], V[b * T:(b + 1) * T])[0] for b in range(B)])


def study(k_bits: np.ndarray, v_bits: np.ndarray, q_bits: np.ndarray, T: int, P: int, C: int, alpha: float,
          splits=(3, 4, 5, 6)) -> dict:
    """vNMSE of the attention outputs of q over K, V reconstructed by each method.

    k_bits, v_bits: [B*T, Hkv, D] BF16 patterns (B sequences of T tokens); q_bits [B, M, Hq, D].
    Keys: 'INT4', 'INT8' (A-linear), 'Lynx' (full decode), 'Lynx-INT4' (anchor only, A-int4),
    'Lynx-INT8 anchor' (A-int8), and 'Lynx anchor a+b' for every split in `splits` (A-split).
    """
    K = o.bf16_bits_to_f64(k_bits)
    V = o.bf16_bits_to_f64(v_bits)
    O = attention_outputs(q_bits, K, V, T)
    res = {}

    def score(name, Kq, Vq):
        res[name] = vnmse(attention_outputs(q_bits, Kq, Vq, T), O)

    score("INT8", linear_roundtrip(K, 8), linear_roundtrip(V, 8))
    score("INT4", linear_roundtrip(K, 4), linear_roundtrip(V, 4))
    score("Lynx-INT8 anchor", int8_split_anchor(K), int8_split_anchor(V))
    kp, Hkv, D = lynx_pages(k_bits, P, C, alpha)
    vp, _, _ = lynx_pages(v_bits, P, C, alpha)
    score("Lynx", lynx_reconstruct(kp, P, Hkv, D, C, alpha, None), lynx_reconstruct(vp, P, Hkv, D, C, alpha, None))
    for a in splits:
        name = "Lynx-INT4" if a == 4 else f"Lynx anchor {a}+{8 - a}"
        score(name, lynx_reconstruct(kp, P, Hkv, D, C, alpha, a), lynx_reconstruct(vp, P, Hkv, D, C, alpha, a))
    return res
