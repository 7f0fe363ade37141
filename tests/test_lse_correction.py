"""CPU model of the 64-row decode's query precision scheme, on the inputs of
the GPU edge cases ``peaked_rows64`` and ``peaked4_rows64``.

The 64-row kernels score the latent part with q_hi = bf16(q_lat) only and add
scale * (q_lo . o) to the log-sum-exp, where q_lo = bf16(q_lat - q_hi) and
o = sum_t p_t c_t under the q_hi scores: the first-order change of
ln sum_t exp(s_t + delta_t) when every latent score gains
delta_t = scale * (q_lo . c_t) (MLA tutorial page, "Position Rotations
Complicate the Absorption": the score is scaled before the softmax).  The
rotary part is multiplied with both bf16 parts.  This test evaluates that
arithmetic in fp64 against the oracle's exact log-sum-exp, at the default
score spread and at 2x and 4x, so the GPU cases are known to sit well inside
the 1e-3 bound before they run, and the uncorrected scheme is shown to miss
it (the cases are sensitive to the correction).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import mla_inputs as M
import oracle.mla_direct as O
from mla_inputs.configs import SegSpec, Spec


def peaked_spec(mul: float) -> Spec:
    return Spec(name=f"edge-peaked-x{mul:g}", batch=4, heads=64, s_q=1, dtype="bf16", d_c=512, d_nope=128,
                d_rope=64, d_v=128, scale=mul / math.sqrt(192),
                segments=(SegSpec("kv", lengths=(1, 37, 300, 1000), online=True),))


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("mul", [1.0, 2.0, 4.0])
def test_first_order_lse_correction(mul):
    x = M.make_inputs(peaked_spec(mul), seed=11)
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    seg = x.segments[0]
    # the query as the decode receives it: fp32 absorption and rotation
    q_lat = O.absorb_query(f(x.w_uk), f(x.q_nope)).astype(np.float32).astype(np.float64)
    q_rot = O.rope_relocate(f(x.q_pe), x.q_pos.numpy(), x.token_shift(seg).numpy(), 10000.0)
    q_rot = q_rot.astype(np.float32).astype(np.float64)
    hi = _bf16(q_lat)
    lo = _bf16(q_lat - hi)
    osegs = [O.OracleSegment(rows=lambda b: f(seg.rows(b)), shift=seg.shift.tolist(), head_begin=0,
                             head_count=x.spec.heads, causal=False)]
    _, _, lse_ref = O.direct_mla_decode(f(x.q_nope), f(x.q_pe), x.q_pos.numpy(), f(x.w_uk), f(x.w_uv), osegs,
                                        x.scale, x.rope_base, 1)
    err_corr = err_plain = 0.0
    for b in range(x.spec.batch):
        rows = f(seg.rows(b))
        c, kr = rows[:, :512], rows[:, 512:]
        for h in range(x.spec.heads):
            s = x.scale * (c @ hi[b, h] + kr @ q_rot[b, h])
            m = s.max()
            lse = m + math.log(np.exp(s - m).sum())
            o = np.exp(s - lse) @ c
            corr = lse + x.scale * float(lo[b, h] @ o)
            err_corr = max(err_corr, abs(corr - lse_ref[b, h]))
            err_plain = max(err_plain, abs(lse - lse_ref[b, h]))
    print(f"spread x{mul:g}: corrected {err_corr:.2e}, uncorrected {err_plain:.2e}")
    assert err_corr <= 2e-4, err_corr          # second order: 5e-6 .. 5e-5 here
    assert err_plain > 1e-3, err_plain         # the case needs the correction
