"""Pins that tie the fp64 oracle to what the pages and mathematics fix.

Each ``pin_*`` takes the oracle module ``O`` and raises AssertionError when the
oracle disagrees with a printed value, a closed form, a library routine or a
brute-force computation written independently here.  ``test_oracle.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` plants plausible mistakes in
a copy of the oracle and checks that some pin fails for every one.
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rot_complex(x, pos, base):
    """RoPE written independently: view pairs (x[2i], x[2i+1]) as the complex
    number x[2i] + i x[2i+1] and multiply by exp(i * pos * base**(-2i/d))."""
    x = list(map(float, x))
    d = len(x)
    out = []
    for i in range(d // 2):
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * pos * base ** (-2.0 * i / d))
        out += [z.real, z.imag]
    return np.array(out)


# ---------------------------------------------------------------- printed values
def pin_worked_example_key_side(O):
    """MLA tutorial page, "The Direct Form Explains the Meaning" and "Move the
    Key Projection Into the Query": U_K c = [1,2,3,-1], score 4 both ways."""
    g = _golden()["key_side"]
    U = np.array(g["up_key"])
    c = np.array(g["latent"])
    q = np.array(g["query"])
    k = O.expand(U, c[None, :])[0]
    _close(k, g["content_key"], 0.0, "U_K c")
    assert float(q @ k) == g["direct_score"]
    qa = O.absorb_query(U[None], q[None, None, :])[0, 0]
    _close(qa, g["absorbed_query"], 0.0, "U_K^T q")
    assert float(qa @ c) == g["absorbed_score"]
    # Through the full single-row attention: one key, scale 1, zero rotary part
    # -> the weight is 1, the lse is the score itself, and o = U_V c.
    o, o_lat, lse = O.attend_direct(q, np.zeros(2), c[None, :], np.zeros((1, 2)), U, U, 1.0)
    assert abs(lse - g["direct_score"]) <= 1e-15, lse
    _close(o, g["content_key"], 1e-15, "o = U_V c for a single key")
    _close(o_lat, c, 1e-15, "o_lat for a single key")


def pin_worked_example_value_side(O):
    """MLA tutorial page, "Move the Value Expansion After the Weighted Sum":
    weights 0.25/0.75 on c1=[1,2], c2=[3,0] give the weighted latent [2.5,0.5]
    and the value output [2.5,0.5,3,2].  The weights are produced by scores
    0 and ln 3 (zero content projection, rotary keys carrying the scores)."""
    g = _golden()["value_side"]
    U = np.array(_golden()["key_side"]["up_key"])
    c = np.array(g["latents"])
    kr = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    o, o_lat, lse = O.attend_direct(np.zeros(4), np.array([1.0, 0.0]), c, kr,
                                    np.zeros((4, 2)), U, 1.0)
    _close(o_lat, g["weighted_latent"], 1e-15, "weighted latent")
    _close(o, g["value_output"], 1e-14, "value output")
    assert abs(lse - math.log(4.0)) <= 1e-15
    # and the output projection call's definition on the weighted latent
    out = O.output_expand(U[None], np.array(g["weighted_latent"])[None, None, :])[0, 0]
    _close(out, g["value_output"], 0.0, "U_V o_lat")
    # expanding first, then mixing, is the same vector (linearity)
    v = O.expand(U, c)
    _close(np.array(g["weights"]) @ v, g["value_output"], 1e-15, "mix of expanded values")


def pin_cache_count(O):
    """MLA tutorial page: 8 bytes per layer-token for d_c = d_r = 2 at two bytes,
    against 32 bytes for two heads of four-number keys and values."""
    g = _golden()["cache_count"]
    assert O.cache_bytes(1, 1, 1, g["mla_d_c"], g["mla_d_r"], g["bytes_per_number"]) == \
        g["mla_bytes_per_token_layer"]
    assert O.mha_cache_bytes(1, 1, 1, g["mha_heads"], g["mha_key_width"], g["mha_value_width"],
                             g["bytes_per_number"]) == g["mha_bytes_per_token_layer"]
    assert O.cache_bytes(61, 64, 32768, 512, 64, 2) == 61 * 64 * 32768 * 576 * 2


# ------------------------------------------------------------- library routines
def _random_head(rng, n, d_c=6, d_nope=5, d_r=4, d_v=3):
    return dict(
        q_nope=rng.standard_normal(d_nope), q_pe=rng.standard_normal(d_r),
        c=rng.standard_normal((n, d_c)), kr=rng.standard_normal((n, d_r)),
        u_k=rng.standard_normal((d_nope, d_c)), u_v=rng.standard_normal((d_v, d_c)))


def pin_vs_torch_sdpa(O):
    """Softmax, scale, mask and LSE: compare with torch's scaled_dot_product_attention
    and logsumexp in fp64 on keys K = [U_K c | rotary key] and values V = U_V c
    built here with torch ops."""
    rng = np.random.default_rng(11)
    for n, scale in ((1, 0.7), (5, 0.3), (37, 1.9)):
        x = _random_head(rng, n)
        pos = 1234
        q_rot = _rot_complex(x["q_pe"], pos, 10000.0)
        o, o_lat, lse = O.attend_direct(x["q_nope"], q_rot, x["c"], x["kr"], x["u_k"], x["u_v"], scale)
        t = {k: torch.tensor(v, dtype=torch.float64) for k, v in x.items()}
        K = torch.cat([t["c"] @ t["u_k"].T, t["kr"]], dim=1)
        Q = torch.cat([t["q_nope"], torch.tensor(q_rot)])
        V = t["c"] @ t["u_v"].T
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None, None, None, :], K[None, None], V[None, None], scale=scale)[0, 0, 0]
        _close(o, ref.numpy(), 1e-12, "o vs sdpa")
        ref_lat = torch.nn.functional.scaled_dot_product_attention(
            Q[None, None, None, :], K[None, None], t["c"][None, None], scale=scale)[0, 0, 0]
        _close(o_lat, ref_lat.numpy(), 1e-12, "o_lat vs sdpa")
        ref_lse = torch.logsumexp(scale * (K @ Q), dim=0).item()
        assert abs(lse - ref_lse) <= 1e-12, (lse, ref_lse)


def pin_masked_vs_torch_sdpa(O):
    """The causal rule (query s of S_q sees rows t <= T - S_q + s) against sdpa
    with an explicit boolean mask, through the whole-step oracle."""
    rng = np.random.default_rng(12)
    T, S_q, H, d_c, d_nope, d_r, d_v = 9, 3, 2, 4, 3, 2, 3
    rows = rng.standard_normal((1, T, d_c + d_r))
    q_nope = rng.standard_normal((S_q, H, d_nope))
    q_pe = rng.standard_normal((S_q, H, d_r))
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    q_pos = np.array([T - S_q + s for s in range(S_q)])
    seg = O.OracleSegment(rows=lambda b: rows[b], shift=[0], head_begin=0, head_count=H, causal=True)
    o, _, lse = O.direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv, [seg], 0.5, 10000.0, S_q)
    c = torch.tensor(rows[0, :, :d_c])
    kr = torch.tensor(rows[0, :, d_c:])  # stored rotary keys are already at their positions
    mask = torch.tensor([[j <= T - S_q + s for j in range(T)] for s in range(S_q)])
    for h in range(H):
        K = torch.cat([c @ torch.tensor(w_uk[h]).T, kr], dim=1)
        V = c @ torch.tensor(w_uv[h]).T
        Q = torch.stack([torch.cat([torch.tensor(q_nope[s, h]),
                                    torch.tensor(_rot_complex(q_pe[s, h], q_pos[s], 10000.0))])
                         for s in range(S_q)])
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None, None], K[None, None], V[None, None], attn_mask=mask, scale=0.5)[0, 0]
        _close(o[:, h], ref.numpy(), 1e-12, f"masked o head {h}")
        sc = 0.5 * (Q @ K.T)
        ref_lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=1)
        _close(lse[:, h], ref_lse.numpy(), 1e-12, f"masked lse head {h}")


# ------------------------------------------------------------- special cases
def pin_special_cases(O):
    rng = np.random.default_rng(13)
    x = _random_head(rng, 1)
    q_rot = rng.standard_normal(4)
    # T = 1: the single weight is 1
    o, o_lat, lse = O.attend_direct(x["q_nope"], q_rot, x["c"], x["kr"], x["u_k"], x["u_v"], 0.8)
    s0 = 0.8 * (x["q_nope"] @ (x["u_k"] @ x["c"][0]) + q_rot @ x["kr"][0])
    assert abs(lse - s0) <= 1e-13
    _close(o, x["u_v"] @ x["c"][0], 1e-13, "T=1 output")
    # identical rows: uniform weights, lse = s + ln T
    n = 7
    c = np.repeat(x["c"], n, axis=0)
    kr = np.repeat(x["kr"], n, axis=0)
    o, o_lat, lse = O.attend_direct(x["q_nope"], q_rot, c, kr, x["u_k"], x["u_v"], 0.8)
    assert abs(lse - (s0 + math.log(n))) <= 1e-13
    _close(o, x["u_v"] @ x["c"][0], 1e-13, "uniform output")
    # very large scale: the weight concentrates on the arg-max row
    y = _random_head(rng, 6)
    s = y["c"] @ y["u_k"].T @ y["q_nope"] + y["kr"] @ q_rot
    o, o_lat, lse = O.attend_direct(y["q_nope"], q_rot, y["c"], y["kr"], y["u_k"], y["u_v"], 1e4)
    _close(o_lat, y["c"][int(np.argmax(s))], 1e-9, "argmax row")
    # no visible row: output 0, lse -inf
    o, o_lat, lse = O.attend_direct(y["q_nope"], q_rot, y["c"][:0], y["kr"][:0], y["u_k"], y["u_v"], 1.0)
    assert lse == -math.inf and not o.any() and not o_lat.any()


def pin_direct_equals_absorbed(O):
    """Regrouping the key projection into the query does not change the score
    (MLA tutorial page, "Move the Key Projection Into the Query")."""
    rng = np.random.default_rng(14)
    H, n_tok, d_nope, d_c = 3, 4, 5, 7
    w = rng.standard_normal((H, d_nope, d_c))
    q = rng.standard_normal((n_tok, H, d_nope))
    c = rng.standard_normal((10, d_c))
    qa = O.absorb_query(w, q)
    for t in range(n_tok):
        for h in range(H):
            direct = O.expand(w[h], c) @ q[t, h]
            _close(direct, c @ qa[t, h], 1e-12, "direct vs absorbed scores")
    # the per-head calls against explicit sums, every head
    w_uv = rng.standard_normal((H, 2, d_c))
    o_lat = rng.standard_normal((n_tok, H, d_c))
    out = O.output_expand(w_uv, o_lat)
    for t in range(n_tok):
        for h in range(H):
            ref_out = [sum(w_uv[h, i, k] * o_lat[t, h, k] for k in range(d_c)) for i in range(2)]
            _close(out[t, h], ref_out, 1e-12, "U_V o_lat explicit sum")
            ref_q = [sum(w[h, i, k] * q[t, h, i] for i in range(d_nope)) for k in range(d_c)]
            _close(qa[t, h], ref_q, 1e-12, "U_K^T q explicit sum")
    # and the output side: U_V (sum a c) = sum a (U_V c)
    a = rng.random(10)
    a /= a.sum()
    for h in range(H):
        mixed = O.output_expand(w_uv[h:h + 1], (a @ c)[None, None, :])[0, 0]
        _close(mixed, a @ O.expand(w_uv[h], c), 1e-12, "value-side linearity")


def pin_output_projection(O):
    """The shared output projection against torch's linear layer (fp64), a
    pure-Python sum, the per-head fold of U_V into W_O (MLA tutorial page,
    "Move the Value Expansion After the Weighted Sum"), and block special
    cases."""
    import torch
    rng = np.random.default_rng(21)
    n_tok, H, d_v, d_c, d_model = 3, 4, 5, 6, 7
    w_o = rng.standard_normal((d_model, H * d_v))
    v = rng.standard_normal((n_tok, H, d_v))
    out = O.output_projection(w_o, v)
    ref = torch.nn.functional.linear(torch.from_numpy(v.reshape(n_tok, H * d_v)), torch.from_numpy(w_o)).numpy()
    _close(out, ref, 1e-12, "W_O vs torch linear")
    for t in range(n_tok):
        for n in range(d_model):
            e = sum(w_o[n, h * d_v + i] * v[t, h, i] for h in range(H) for i in range(d_v))
            assert abs(out[t, n] - e) <= 1e-12, "W_O explicit sum"
    # the fold: (W_O block h . U_V[h]) o_lat[h], summed over heads, equals
    # W_O applied to the expanded heads
    w_uv = rng.standard_normal((H, d_v, d_c))
    o_lat = rng.standard_normal((n_tok, H, d_c))
    fold = O.fold_value_into_output(w_o, w_uv)
    assert fold.shape == (H, d_model, d_c)
    via_fold = sum(o_lat[:, h, :] @ fold[h].T for h in range(H))
    expanded = np.einsum("hvc,thc->thv", w_uv, o_lat)
    ref2 = torch.nn.functional.linear(torch.from_numpy(expanded.reshape(n_tok, H * d_v)),
                                      torch.from_numpy(w_o)).numpy()
    _close(via_fold, ref2, 1e-12, "folded U_V W_O")
    # one head with W_O = identity passes the head's output through; W_O
    # nonzero only on head 2's columns sees head 2 alone
    v1 = rng.standard_normal((2, 1, d_v))
    _close(O.output_projection(np.eye(d_v), v1), v1[:, 0, :], 1e-15, "identity W_O")
    w_blk = np.zeros_like(w_o)
    w_blk[:, 2 * d_v:3 * d_v] = w_o[:, 2 * d_v:3 * d_v]
    _close(O.output_projection(w_blk, v), v[:, 2, :] @ w_o[:, 2 * d_v:3 * d_v].T, 1e-12, "single head block")


# ------------------------------------------------------------------- RoPE
def pin_rope(O):
    rng = np.random.default_rng(15)
    base = 10000.0
    d = 8
    x = rng.standard_normal(d)
    y = rng.standard_normal(d)
    # against the complex-number formulation (fixes pairing, sign and frequencies)
    for pos in (0, 1, 7, 4095, 262143):
        _close(O.rope_rotate(x, pos, base), _rot_complex(x, pos, base), 1e-9, f"rope at {pos}")
    # R(0) = I, norm preserved, (R(a)x).(R(b)y) = x.(R(b-a)y)
    _close(O.rope_rotate(x, 0, base), x, 0.0, "R(0)")
    assert abs(np.linalg.norm(O.rope_rotate(x, 99991, base)) - np.linalg.norm(x)) <= 1e-12
    for a, b in ((3, 10), (1000, 123456), (220000, 219000)):
        lhs = O.rope_rotate(x, a, base) @ O.rope_rotate(y, b, base)
        rhs = x @ O.rope_rotate(y, b - a, base)
        assert abs(lhs - rhs) <= 1e-10, (a, b, lhs, rhs)
    # the first pair rotates by exactly pos radians
    e = np.zeros(d)
    e[0] = 1.0
    r = O.rope_rotate(e, 2.0, base)
    _close(r[:2], [math.cos(2.0), math.sin(2.0)], 1e-15, "first pair")
    # relocation = rotation by (pos - shift)
    q = rng.standard_normal((3, 2, d))
    pos = np.array([5, 200000, 262143])
    shift = np.array([5, 1234, 0])
    rq = O.rope_relocate(q, pos, shift, base)
    for t in range(3):
        for h in range(2):
            _close(rq[t, h], _rot_complex(q[t, h], int(pos[t] - shift[t]), base), 1e-9, "relocate")


def pin_relocation_invariance(O):
    """A segment stored at canonical positions 0..n-1 and read with shift o
    equals the same keys stored at their true positions o..o+n-1 (rotated here
    independently) and read with shift 0 (RedKnot-MLA abstract: relocating the
    query restores the document's request position)."""
    rng = np.random.default_rng(16)
    n, H, d_c, d_nope, d_r, d_v = 11, 2, 4, 3, 4, 2
    o_b = 187_345
    raw = rng.standard_normal((1, n, d_c + d_r))
    stored_canon = raw.copy()
    stored_canon[0, :, d_c:] = np.stack([_rot_complex(raw[0, j, d_c:], j, 1e4) for j in range(n)])
    stored_true = raw.copy()
    stored_true[0, :, d_c:] = np.stack([_rot_complex(raw[0, j, d_c:], o_b + j, 1e4) for j in range(n)])
    q_nope = rng.standard_normal((1, H, d_nope))
    q_pe = rng.standard_normal((1, H, d_r))
    q_pos = np.array([o_b + n + 40])
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    a = O.direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv,
                            [O.OracleSegment(lambda b: stored_canon[b], [o_b], 0, H, False)],
                            0.4, 1e4, 1)
    b = O.direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv,
                            [O.OracleSegment(lambda b: stored_true[b], [0], 0, H, False)],
                            0.4, 1e4, 1)
    for x, y, what in zip(a, b, ("o", "o_lat", "lse")):
        _close(x, y, 1e-9, f"relocation {what}")


# ----------------------------------------------------------------- merge
def pin_segment_merge(O):
    """merge(partial(A), partial(B)) equals one softmax over A and B."""
    rng = np.random.default_rng(17)
    x = _random_head(rng, 23)
    q_rot = rng.standard_normal(4)
    full = O.attend_direct(x["q_nope"], q_rot, x["c"], x["kr"], x["u_k"], x["u_v"], 0.6)
    for cuts in ((0, 10, 23), (0, 1, 2, 23), (0, 23, 23), (0, 5, 5, 17, 23)):
        parts = [O.attend_direct(x["q_nope"], q_rot, x["c"][a:b], x["kr"][a:b], x["u_k"], x["u_v"], 0.6)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = O.merge_lse(np.stack([p[1] for p in parts]), np.array([p[2] for p in parts]))
        _close(o, full[1], 1e-12, f"merged o_lat {cuts}")
        assert abs(lse - full[2]) <= 1e-12
        ov, _ = O.merge_lse(np.stack([p[0] for p in parts]), np.array([p[2] for p in parts]))
        _close(ov, full[0], 1e-12, f"merged o {cuts}")
    # closed forms: two equal states -> same o, lse + ln 2; all empty -> (0, -inf)
    o, lse = O.merge_lse(np.stack([full[1], full[1]]), np.array([full[2], full[2]]))
    _close(o, full[1], 1e-14, "equal merge")
    assert abs(lse - (full[2] + math.log(2.0))) <= 1e-13
    o, lse = O.merge_lse(np.zeros((3, 4)), np.full(3, -math.inf))
    assert lse == -math.inf and not o.any()
    # a NaN payload behind an empty slot is never read
    o, lse = O.merge_lse(np.stack([full[1], np.full_like(full[1], np.nan)]),
                         np.array([full[2], -math.inf]))
    _close(o, full[1], 0.0, "empty slot skipped")


# -------------------------------------------------------------- brute force
def _brute(q_nope, q_pe, q_pos, w_uk, w_uv, segs, scale, base, s_q):
    """Pure-Python loops: expand, rotate, score, softmax, weight."""
    n_tok, H, d_nope = len(q_nope), len(q_nope[0]), len(q_nope[0][0])
    d_c = len(w_uk[0][0])
    d_v = len(w_uv[0])
    out = [[None] * H for _ in range(n_tok)]
    lses = [[None] * H for _ in range(n_tok)]
    for t in range(n_tok):
        b, s = divmod(t, s_q)
        for h in range(H):
            scores, vals = [], []
            for (rows, shift, h0, hc, causal) in segs:
                if not (h0 <= h < h0 + hc):
                    continue
                rb = rows[b]
                T = len(rb)
                for j in range(T):
                    if causal and j > T - s_q + s:
                        continue
                    c = rb[j][:d_c]
                    kr = _rot_complex(rb[j][d_c:], shift[b], base)
                    qr = _rot_complex(q_pe[t][h], q_pos[t], base)
                    sc = 0.0
                    for i in range(d_nope):
                        sc += q_nope[t][h][i] * sum(w_uk[h][i][k] * c[k] for k in range(d_c))
                    for i in range(len(kr)):
                        sc += qr[i] * kr[i]
                    scores.append(scale * sc)
                    vals.append([sum(w_uv[h][i][k] * c[k] for k in range(d_c)) for i in range(d_v)])
            if not scores:
                out[t][h] = [0.0] * d_v
                lses[t][h] = -math.inf
                continue
            m = max(scores)
            den = sum(math.exp(x - m) for x in scores)
            out[t][h] = [sum(math.exp(scores[j] - m) / den * vals[j][i] for j in range(len(vals)))
                         for i in range(d_v)]
            lses[t][h] = m + math.log(den)
    return np.array(out), np.array(lses)


def pin_brute_force(O):
    """Two segments with head ranges and a causal segment, shifts, S_q = 2."""
    rng = np.random.default_rng(18)
    B, S_q, H, d_c, d_nope, d_r, d_v = 2, 2, 3, 3, 2, 4, 2
    rows_a = [rng.standard_normal((n, d_c + d_r)) for n in (4, 0)]
    rows_b = [rng.standard_normal((n, d_c + d_r)) for n in (3, 5)]
    rows_c = [rng.standard_normal((n, d_c + d_r)) for n in (2, 6)]
    q_nope = rng.standard_normal((B * S_q, H, d_nope))
    q_pe = rng.standard_normal((B * S_q, H, d_r))
    q_pos = np.array([40, 41, 17, 18])
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    segs = [(rows_a, [7, 3], 0, 2, False), (rows_b, [0, 0], 2, 1, False), (rows_c, [0, 0], 0, 3, True)]
    o, _, lse = O.direct_mla_decode(
        q_nope, q_pe, q_pos, w_uk, w_uv,
        [O.OracleSegment(lambda b, r=r: r[b], sh, h0, hc, ca) for (r, sh, h0, hc, ca) in segs],
        0.45, 10000.0, S_q)
    ob, lb = _brute(q_nope.tolist(), q_pe.tolist(), q_pos.tolist(), w_uk.tolist(), w_uv.tolist(),
                    [([x.tolist() for x in r], sh, h0, hc, ca) for (r, sh, h0, hc, ca) in segs],
                    0.45, 10000.0, S_q)
    _close(o, ob, 1e-12, "brute-force o")
    _close(lse, lb, 1e-12, "brute-force lse")


# ------------------------------------------------------------------ QK-Norm
def pin_qknorm_closed_form(O):
    """QK-Norm MLA page (abstract), RMSNorm(x) = g x / sqrt(mean(x^2) + eps):
    one head and one key with the tutorial's teaching numbers (U_K c =
    [1,2,3,-1], q = [1,0,1,0], q . k = 4): the content score is
    (g_q q . g_k k) / (sqrt(|q|^2/4 + eps) sqrt(|k|^2/4 + eps)), derived by hand."""
    g = _golden()["key_side"]
    U = np.array(g["up_key"])[None]           # [1, 4, 2]
    c = np.array(g["latent"])[None, :]        # one row
    q = np.array(g["query"])[None, None, :]   # one token, one head
    rows = np.concatenate([c, np.zeros((1, 2))], axis=1)   # zero rotary key
    seg = [O.OracleSegment(lambda b: rows, [0], 0, 1, False)]

    def lse_of(g_q, g_k, eps):
        qk = O.QKNorm(np.array([g_q], float), np.array([g_k], float), eps)
        _, _, lse = O.direct_mla_decode(q, np.zeros((1, 1, 2)), np.array([0]), U, U, seg, 1.0, 10000.0, 1,
                                        qk_norm=qk)
        return float(lse[0, 0])

    # |q|^2 = 2, |k|^2 = 15
    assert abs(lse_of([1, 1, 1, 1], [1, 1, 1, 1], 0.0) - 16.0 / math.sqrt(30.0)) <= 1e-14
    assert abs(lse_of([1, 1, 1, 1], [1, 1, 1, 1], 0.5) - 4.0 / math.sqrt(4.25)) <= 1e-14
    # g_q * g_k weights the terms q_i k_i: 2*1*1*1 (i=0) + 1*0.5*1*3 (i=2) = 3.5
    assert abs(lse_of([2, 1, 1, 1], [1, 1, 0.5, 1], 0.0) - 3.5 / math.sqrt(0.5 * 3.75)) <= 1e-14


def pin_qknorm_invariances(O):
    """With eps = 0 the normalised content scores ignore positive rescaling of a
    token's whole query (all heads) and of any latent row: the lse is unchanged,
    and scaling every latent of a request scales o and o_lat by the same
    factor (values stay linear in c)."""
    rng = np.random.default_rng(21)
    B, S_q, H, d_c, d_nope, d_r, d_v = 1, 2, 3, 5, 4, 2, 3
    rows = rng.standard_normal((6, d_c + d_r))
    q_nope = rng.standard_normal((B * S_q, H, d_nope))
    q_pe = rng.standard_normal((B * S_q, H, d_r))
    q_pos = np.array([9, 10])
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    qk = O.QKNorm(1.0 + 0.3 * rng.standard_normal((H, d_nope)), 1.0 + 0.3 * rng.standard_normal((H, d_nope)), 0.0)

    def run(r, q):
        return O.direct_mla_decode(q, q_pe, q_pos, w_uk, w_uv, [O.OracleSegment(lambda b: r, [0], 0, H, True)],
                                   0.7, 10000.0, S_q, qk_norm=qk)

    o, o_lat, lse = run(rows, q_nope)
    q2 = q_nope.copy()
    q2[1] *= 3.7                                        # one whole token
    o2, _, lse2 = run(rows, q2)
    _close(lse2, lse, 1e-12, "query rescaling: lse")
    _close(o2, o, 1e-12, "query rescaling: o")
    r2 = rows.copy()
    r2[2, :d_c] *= 0.25                                 # one latent row
    _, _, lse3 = run(r2, q_nope)
    _close(lse3, lse, 1e-12, "latent row rescaling: lse")
    r3 = rows.copy()
    r3[:, :d_c] *= 2.5                                  # every latent row
    o4, o_lat4, lse4 = run(r3, q_nope)
    _close(lse4, lse, 1e-12, "latent rescaling: lse")
    _close(o4, 2.5 * o, 1e-12, "latent rescaling: o")
    _close(o_lat4, 2.5 * o_lat, 1e-12, "latent rescaling: o_lat")


def pin_qknorm_absorbed(O):
    """QK-Norm MLA page (abstract): the static key weight moves into the query
    projection and the key statistic becomes one inverse-RMS scalar per row.
    The absorbed form is written here from that statement: q' = U_K^T (g_q g_k
    q) / rms(q) per head, r_t = 1 / sqrt(c_t^T M c_t / (H d_nope) + eps) with
    M = sum_h U_K[h]^T U_K[h] (a quadratic form, no key expansion), score =
    scale (r_t q'.c_t + q_rot.kr_t); it must equal the oracle's explicit form."""
    rng = np.random.default_rng(22)
    B, S_q, H, d_c, d_nope, d_r, d_v = 2, 2, 3, 6, 4, 4, 3
    rows = [rng.standard_normal((n, d_c + d_r)) for n in (7, 4)]
    q_nope = rng.standard_normal((B * S_q, H, d_nope))
    q_pe = rng.standard_normal((B * S_q, H, d_r))
    q_pos = np.array([30, 31, 12, 13])
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    eps, scale, base = 0.3, 0.55, 10000.0
    qk = O.QKNorm(1.0 + 0.2 * rng.standard_normal((H, d_nope)), 1.0 + 0.2 * rng.standard_normal((H, d_nope)), eps)
    o, _, lse = O.direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv,
                                    [O.OracleSegment(lambda b: rows[b], [0, 0], 0, H, True)],
                                    scale, base, S_q, qk_norm=qk)
    M = sum(w_uk[h].T @ w_uk[h] for h in range(H))
    for b in range(B):
        c, kr = rows[b][:, :d_c], rows[b][:, d_c:]
        T = c.shape[0]
        r = 1.0 / np.sqrt(np.einsum("nd,de,ne->n", c, M, c) / (H * d_nope) + eps)
        for s in range(S_q):
            t = b * S_q + s
            rq = 1.0 / math.sqrt(float(np.mean(q_nope[t] ** 2)) + eps)
            vis = T - S_q + s + 1
            krot = np.array([_rot_complex(kr[j], 0, base) for j in range(vis)])
            for h in range(H):
                qa = w_uk[h].T @ (qk.g_q[h] * qk.g_k[h] * q_nope[t, h]) * rq
                qr = np.array(_rot_complex(q_pe[t, h], q_pos[t], base))
                sc = scale * (r[:vis] * (c[:vis] @ qa) + krot @ qr)
                m = sc.max()
                a = np.exp(sc - m)
                ref_lse = m + math.log(a.sum())
                ref_o = (a / a.sum()) @ (c[:vis] @ w_uv[h].T)
                assert abs(lse[t, h] - ref_lse) <= 1e-12, (t, h, lse[t, h], ref_lse)
                _close(o[t, h], ref_o, 1e-12, "absorbed QK-Norm o")


ALL_PINS = [
    pin_worked_example_key_side,
    pin_worked_example_value_side,
    pin_cache_count,
    pin_vs_torch_sdpa,
    pin_masked_vs_torch_sdpa,
    pin_special_cases,
    pin_direct_equals_absorbed,
    pin_rope,
    pin_relocation_invariance,
    pin_segment_merge,
    pin_brute_force,
    pin_qknorm_closed_form,
    pin_qknorm_invariances,
    pin_qknorm_absorbed,
    pin_output_projection,
]
