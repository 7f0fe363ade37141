"""Shared helpers of the GPU parity tests: oracle calls on the seeded inputs
and the tolerance checks.

Tolerances (from the decode target): bf16 workloads
  max|o - o_ref| <= 1e-2 * max|o_ref| + 1e-3   and   max|lse - lse_ref| <= 1e-3;
fp32 toy
  max|o - o_ref| <= 1e-5 * max|o_ref|   and   |lse - lse_ref| <= 1e-5 * max(1, |lse_ref|).
The output bound is taken per request: max|o_ref| runs over that request's
own query tokens and heads, so a short request with large outputs (a one-row
request returns its row's value) does not loosen the bound on long ones.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.mla_direct as O
import oracle.mla_quant as Q


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_rows(x, seg, b):
    """Rows of request b as attention reads them: the stored bf16 rows, or
    with an int8 cache the oracle's own quantize/dequantize of their latents."""
    r = f64(seg.rows(b))
    if x.spec.quant == "int8":
        r = Q.quantized_rows(seg.rows(b).float().numpy(), x.spec.d_c)
    elif x.spec.quant == "int4":
        r = Q.quantized_rows_i4(seg.rows(b).float().numpy(), x.spec.d_c)
    return r


def oracle_segments(x):
    return [O.OracleSegment(rows=(lambda b, s=s: oracle_rows(x, s, b)), shift=s.shift.tolist(),
                            head_begin=s.head_begin, head_count=s.head_count, causal=s.causal)
            for s in x.segments]


def oracle_decode(x, requests=None, heads=None):
    """(o, o_lat, lse) of the direct form for the given requests/heads (NaN elsewhere)."""
    qk = O.QKNorm(f64(x.g_q), f64(x.g_k), x.spec.qk_eps) if x.g_q is not None else None
    return O.direct_mla_decode(f64(x.q_nope), f64(x.q_pe), x.q_pos.numpy(), f64(x.w_uk), f64(x.w_uv),
                               oracle_segments(x), x.scale, x.rope_base, x.spec.s_q,
                               requests=requests, heads=heads, qk_norm=qk)


def tol_check(name, got, ref, fp32: bool, kind: str, mask=None, s_q: int = 0):
    """Assert the decode tolerance on the entries where mask (or ref) is set.
    kind: 'o' (outputs, relative to max|ref|) or 'lse'.  With s_q > 0 the
    first axis is the query token (request b owns tokens b*s_q .. b*s_q+s_q-1)
    and the output bound is checked request by request."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if kind == "o" and s_q > 0 and mask is None:
        n_req = ref.shape[0] // s_q
        worst = 0.0
        for b in range(n_req):
            r = ref[b * s_q:(b + 1) * s_q]
            if np.all(np.isnan(r)):
                continue
            worst = max(worst, tol_check(f"{name} request {b}", got[b * s_q:(b + 1) * s_q], r, fp32, "o"))
        return worst
    sel = ~np.isnan(ref) if mask is None else mask
    g, r = got[sel], ref[sel]
    assert g.size > 0, f"{name}: nothing to compare"
    if kind == "lse":
        both_inf = np.isneginf(r) & np.isneginf(g)
        assert np.array_equal(np.isneginf(r), np.isneginf(g)), f"{name}: -inf pattern differs"
        g, r = g[~both_inf], r[~both_inf]
        if g.size == 0:
            return 0.0
        err = np.abs(g - r)
        bound = 1e-5 * np.maximum(1.0, np.abs(r)) if fp32 else np.full_like(r, 1e-3)
        worst = float(np.max(err - bound))
        assert np.all(np.isfinite(g)), f"{name}: non-finite lse"
        assert worst <= 0, f"{name}: lse err {float(np.max(err)):.3e} exceeds bound by {worst:.3e}"
        return float(np.max(err))
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = float(np.max(np.abs(g - r)))
    scale = float(np.max(np.abs(r)))
    bound = 1e-5 * scale if fp32 else 1e-2 * scale + 1e-3
    if fp32:
        bound = max(bound, 1e-30)
    assert err <= bound, f"{name}: max abs err {err:.3e} > bound {bound:.3e} (max|ref| {scale:.3e})"
    return err


def check_step(x, out, o_lat, lse, requests=None, heads=None, label=""):
    """Compare a GPU step's (out, o_lat, lse) with the oracle on (requests x heads)."""
    fp32 = x.spec.dtype == "f32"
    o_ref, lat_ref, lse_ref = oracle_decode(x, requests, heads)
    s_q = x.spec.s_q
    errs = {
        "o": tol_check(f"{label} out", f64(out), o_ref, fp32, "o", s_q=s_q),
        "o_lat": tol_check(f"{label} o_lat", f64(o_lat), lat_ref, fp32, "o", s_q=s_q),
        "lse": tol_check(f"{label} lse", f64(lse), lse_ref, fp32, "lse"),
    }
    return errs


def sample_pairs(x, n_req: int, n_head: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    B, H = x.spec.batch, x.spec.heads
    reqs = sorted(rng.choice(B, size=min(n_req, B), replace=False).tolist())
    heads = sorted(set(rng.choice(H, size=min(n_head, H), replace=False).tolist()) | {0, H - 1})
    return reqs, heads
