"""Element-by-element comparison of the GPU codec's streams with the oracle.

Contract (written out here, used by every GPU parity test):
  metadata  gamma_min, gamma_scale bit-exact.  mu, sigma bit-exact except a
            1-ulp float32 difference where the oracle's float64 value lies within
            1e-12 (relative) of the float32 rounding midpoint between the two.
  codes     compared with the oracle's Stages 2-4 run on the GPU's stored
            metadata; identical except <= 1e-4 of elements differing by 1 in the
            7-bit code I, and only where |Y_oracle - (k + 1/2)| < 1e-6.
  decode    float32 output: max |gpu - oracle_decode(same codes, same metadata)|
            <= 1e-3 * (gamma_scale + eps) of the channel (page scale).  BF16 output: the
            correctly rounded BF16 of a value within the float32 evaluation bound of
            the oracle value (2^-21 (|x_hat| + |gamma_min + mu D1|)); the share of
            outputs that differ from the correctly rounded oracle value is reported.
"""
from __future__ import annotations

import numpy as np

from oracle import lynx_oracle as o

CODE_FLIP_FRAC = 1e-4
CODE_BAND = 1e-6
META_MID_REL = 1e-12
DECODE_REL_SCALE = 1e-3


def _f32_next(a, direction):
    return np.nextafter(a.astype(np.float32), np.float32(direction), dtype=np.float32)


def check_metadata(got: dict, enc: dict, X: np.ndarray, C: int, report: dict):
    """got: parsed GPU anchor segment; enc: oracle encode of the same page."""
    for key in ("gmin", "gscale"):
        bad = np.nonzero(got[key].view(np.uint32) != enc[key].view(np.uint32))[0]
        assert bad.size == 0, (f"{key} differs at channels {bad[:8].tolist()}: gpu {got[key][bad[:8]].tolist()} "
                               f"oracle {enc[key][bad[:8]].tolist()}")
    mu_g, mu_o = got["mu"], enc["mu"]
    bad = mu_g.view(np.uint32) != mu_o.view(np.uint32)
    if bad.any():
        mid = (mu_g[bad].astype(np.float64) + mu_o[bad].astype(np.float64)) / 2
        one_ulp = (mu_g[bad] == _f32_next(mu_o[bad], np.inf)) | (mu_g[bad] == _f32_next(mu_o[bad], -np.inf))
        near = np.abs(enc["mu64"][bad] - mid) <= META_MID_REL * np.abs(enc["mu64"][bad])
        assert np.all(one_ulp & near), f"mu differs beyond the midpoint exemption at {bad.sum()} entries"
    report["mu_ulp_flips"] = report.get("mu_ulp_flips", 0) + int(bad.sum())
    # sigma against the oracle's definition evaluated with the GPU's stored mu
    Xn = o.normalize_page(X, got["gmin"], got["gscale"])
    sig_ref = o.chunk_sigma(Xn, got["mu"], C)
    dev64 = np.abs(o.chunk_view(Xn, C) - got["mu"].astype(np.float64)[:, None, :]).max(axis=1)
    sbad = got["sigma"].view(np.uint32) != sig_ref.view(np.uint32)
    if sbad.any():
        mid = (got["sigma"][sbad].astype(np.float64) + sig_ref[sbad].astype(np.float64)) / 2
        near = np.abs(dev64[sbad] - mid) <= META_MID_REL * np.abs(dev64[sbad])
        assert np.all(near), f"sigma differs beyond the midpoint exemption at {sbad.sum()} entries"
    report["sigma_ulp_flips"] = report.get("sigma_ulp_flips", 0) + int(sbad.sum())


def check_codes(got: dict, q_res_gpu, X: np.ndarray, C: int, alpha: float, report: dict):
    """Codes of one page against the oracle run on the GPU's stored metadata."""
    ref = o.codes_given_metadata(X, got["gmin"], got["gscale"], got["mu"], got["sigma"], C, alpha)
    ga = got["Q_anc"]
    same_anc = ga == ref["Q_anc"]
    if q_res_gpu is not None:
        S_g, I_g = o.code_full(ga, q_res_gpu)
        diff = (I_g != ref["I"]) | (S_g != ref["S"])
        if diff.any():
            Y = ref["Y"][diff]
            assert np.all(S_g[diff] == ref["S"][diff]), "sign differs"
            assert np.all(np.abs(I_g[diff] - ref["I"][diff]) == 1), "code differs by more than 1"
            assert np.all(np.abs(Y - np.floor(Y) - 0.5) < CODE_BAND), "code flip away from a rounding boundary"
        report["code_flips"] = report.get("code_flips", 0) + int(diff.sum())
    else:
        diff = ~same_anc
        if diff.any():
            Y = ref["Y"][diff]
            assert np.all(np.abs(Y - np.floor(Y) - 0.5) < CODE_BAND), "anchor flip away from a rounding boundary"
        report["code_flips"] = report.get("code_flips", 0) + int(diff.sum())
    report["elements"] = report.get("elements", 0) + ga.size


def finish_codes(report: dict):
    assert report["code_flips"] <= CODE_FLIP_FRAC * report["elements"], report


def check_decode_f32(out_f32: np.ndarray, ref64: np.ndarray, gscale: np.ndarray, report: dict):
    """out_f32 / ref64: [P, H] of one page; gscale: [H] float32 of the page."""
    err = np.abs(out_f32.astype(np.float64) - ref64).max(axis=0)
    # page scale = gamma_scale + eps, the Stage 1 divisor (equal to gamma_scale for any channel
    # whose range is not below eps)
    scale = gscale.astype(np.float64) + o.EPS
    bound = DECODE_REL_SCALE * scale
    assert np.all(err <= bound), f"decode error {np.max(err / bound):.3g} x bound"
    report["decode_max_rel_scale"] = max(report.get("decode_max_rel_scale", 0.0), float(np.max(err / scale)))


def decode_slack(got: dict, ref64: np.ndarray, C: int) -> np.ndarray:
    """Per-element bound on a float32 evaluation of x_hat = A*L + B (A, L, B each rounded to
    float32, one fused multiply-add): 2^-21 * (|x_hat| + |B|), with B = gamma_min + mu*D1."""
    P, H = ref64.shape
    D1 = got["gscale"].astype(np.float64) + o.EPS
    Bc = got["gmin"].astype(np.float64)[None, :] + got["mu"].astype(np.float64) * D1[None, :]
    B = np.repeat(Bc, C, axis=0)
    return 2.0 ** -21 * (np.abs(ref64) + np.abs(B))


def check_decode_bf16(out_bits: np.ndarray, ref64: np.ndarray, slack: np.ndarray, report: dict):
    """BF16 output must be a correctly rounded BF16 of some value within `slack` of the
    oracle value: round(ref - slack) <= out <= round(ref + slack)."""
    out = o.bf16_bits_to_f64(out_bits)
    lo = o.bf16_bits_to_f64(o.f64_to_bf16_bits(ref64 - slack))
    hi = o.bf16_bits_to_f64(o.f64_to_bf16_bits(ref64 + slack))
    ok = (out >= lo) & (out <= hi)
    assert np.all(ok), f"BF16 output outside the rounding bracket at {int((~ok).sum())} elements"
    exact = out_bits == o.f64_to_bf16_bits(ref64)
    report["bf16_flips"] = report.get("bf16_flips", 0) + int((~exact).sum())
    report["bf16_elements"] = report.get("bf16_elements", 0) + out_bits.size


def finish_bf16(report: dict, max_share: float | None = CODE_FLIP_FRAC):
    """Outputs that differ from the correctly rounded oracle value lie inside the float32
    bracket (checked per element); on the synthetic KV their share stays below 1e-4.
    Degenerate pages built to force cancellation pass max_share=None."""
    if max_share is not None:
        assert report["bf16_flips"] <= max_share * report["bf16_elements"], report
