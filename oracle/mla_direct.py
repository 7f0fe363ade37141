"""Direct-form MLA decode in fp64 on the CPU: the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this file; it is used by the tests, by the smoke check and by the benchmark's
CPU-baseline leg.  It shares no code with the HIP library.

Everything here is the *plain definition* of what absorbed MLA decode reaches
by regrouping.  Sources (the pages' titles and sections):

* "Multi-Head Latent Attention: How DeepSeek Compressed the Cache Further"
  (the MLA tutorial page):
  - "Learn a Smaller Shared Representation": per-head up-projections turn the
    shared latent into the content key and the value (k_t = U_K c_t,
    v_t = U_V c_t, with U mapping the small vector to the wider one);
  - "The Direct Form Explains the Meaning": expand the key, then dot it with
    the query;
  - "Move the Value Expansion After the Weighted Sum": the ordinary weighted
    sum of expanded values, and the weighted latent;
  - "Position Rotations Complicate the Absorption": the score is the content
    score plus a position score from a separate rotary key; the sum is scaled
    and masked, then softmaxed;
  - "Count the Cache That Is Actually Stored": bytes per stored entry.
* "RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4 Long-Context
  Serving" (abstract): a document cached at canonical position zero is read at
  its true request position; partial results of separate paths are merged
  before one shared output projection.
* The QK-Norm MLA page (abstract): query-key RMSNorm after the projections,
  RMSNorm = a static weight times x over a dynamic root-mean-square.

Readings taken where the pages are silent (each also listed in the design
notes): RoPE rotates adjacent feature pairs (2i, 2i+1) counter-clockwise by
angle pos * base**(-2i/d_rope); the softmax scale is a parameter; a query row
with no visible key gives output 0 and log-sum-exp -inf; the log-sum-exp is
the natural logarithm; under a causal rule query ``s`` of ``S_q`` sees rows
``t <= T - S_q + s`` of that segment.

Here the key is moved to its *true* position (key-side); the GPU path rotates
the query instead (query-side).  The two agree only because rotations
compose, which is what the tests check.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence

import numpy as np

NEG_INF = -math.inf


# --------------------------------------------------------------------------
# Rotary position embedding ("Position Rotations Complicate the Absorption")
# --------------------------------------------------------------------------
def rope_frequencies(d_rope: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2 i / d_rope) for the d_rope/2 feature pairs."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return base ** (-2.0 * i / d_rope)


def rope_rotate(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each adjacent pair (x[2i], x[2i+1]) of the last axis by the angle
    pos * theta_i, counter-clockwise:  (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).

    ``pos`` broadcasts against ``x[..., 0]`` (integer positions, exact in fp64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = rope_frequencies(d, base)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def rope_relocate(q_pe: np.ndarray, pos: np.ndarray, shift: np.ndarray, base: float) -> np.ndarray:
    """Query-side relocation: rotate the unrotated query part by (pos - shift).

    q_pe [n_tok, H, d_rope]; pos, shift integer [n_tok].  With shift = 0 this is
    ordinary query RoPE at the true position (RedKnot-MLA abstract: the query is
    moved instead of re-rotating the cached keys)."""
    rel = np.asarray(pos, dtype=np.int64) - np.asarray(shift, dtype=np.int64)
    return rope_rotate(q_pe, rel[:, None], base)


# --------------------------------------------------------------------------
# Up-projections ("Learn a Smaller Shared Representation", "The Direct Form")
# --------------------------------------------------------------------------
def expand(U: np.ndarray, c: np.ndarray) -> np.ndarray:
    """U c_t for every row: U [d_out, d_c], c [n, d_c] -> [n, d_out]."""
    return np.asarray(c, dtype=np.float64) @ np.asarray(U, dtype=np.float64).T


def absorb_query(w_uk: np.ndarray, q_nope: np.ndarray) -> np.ndarray:
    """The per-head query transform U_K^T q ("Move the Key Projection Into the
    Query"): w_uk [H, d_nope, d_c], q_nope [n_tok, H, d_nope] -> [n_tok, H, d_c].
    This is the plain definition of the absorption call, used to check it."""
    w = np.asarray(w_uk, dtype=np.float64)
    q = np.asarray(q_nope, dtype=np.float64)
    out = np.empty(q.shape[:2] + (w.shape[2],), dtype=np.float64)
    for h in range(w.shape[0]):
        out[:, h, :] = q[:, h, :] @ w[h]
    return out


def output_expand(w_uv: np.ndarray, o_lat: np.ndarray) -> np.ndarray:
    """out = U_V o_lat per head: w_uv [H, d_v, d_c], o_lat [n_tok, H, d_c] -> [n_tok, H, d_v]."""
    w = np.asarray(w_uv, dtype=np.float64)
    o = np.asarray(o_lat, dtype=np.float64)
    out = np.empty(o.shape[:2] + (w.shape[1],), dtype=np.float64)
    for h in range(w.shape[0]):
        out[:, h, :] = o[:, h, :] @ w[h].T
    return out


def output_projection(w_o: np.ndarray, v: np.ndarray) -> np.ndarray:
    """The shared output projection over the heads' value outputs: each head
    adds its own contribution, the columns of W_O that belong to it applied to
    that head's d_v outputs (MLA tutorial page, "Move the Value Expansion After
    the Weighted Sum", its closing remark that U_V combines with the head's
    contribution to the final output projection; RedKnot-MLA abstract: one
    shared output projection after the merge).

    w_o [d_model, H * d_v] (head h owns columns h*d_v .. h*d_v + d_v - 1),
    v [n_tok, H, d_v] -> [n_tok, d_model]."""
    w = np.asarray(w_o, dtype=np.float64)
    x = np.asarray(v, dtype=np.float64)
    n_tok, H, d_v = x.shape
    out = np.zeros((n_tok, w.shape[0]), dtype=np.float64)
    for h in range(H):
        out += x[:, h, :] @ w[:, h * d_v:(h + 1) * d_v].T
    return out


def fold_value_into_output(w_o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """W_O's columns of head h times that head's U_V: one [d_model, d_c] map per
    head that takes the weighted latent straight to the head's share of the
    layer output (the same remark of the MLA tutorial page).

    w_o [d_model, H * d_v], w_uv [H, d_v, d_c] -> [H, d_model, d_c]."""
    w = np.asarray(w_o, dtype=np.float64)
    u = np.asarray(w_uv, dtype=np.float64)
    H, d_v, d_c = u.shape
    return np.stack([w[:, h * d_v:(h + 1) * d_v] @ u[h] for h in range(H)])


# --------------------------------------------------------------------------
# Softmax with its log-sum-exp
# --------------------------------------------------------------------------
def softmax_lse(scores: np.ndarray):
    """Ordinary two-pass softmax of a 1-D score vector: (weights, natural-log LSE).
    An empty vector gives (empty, -inf)."""
    s = np.asarray(scores, dtype=np.float64)
    if s.size == 0:
        return s.copy(), NEG_INF
    m = s.max()
    e = np.exp(s - m)
    tot = e.sum()
    return e / tot, float(m + math.log(tot))


def attend_direct(q_nope: np.ndarray, q_rot: np.ndarray, c: np.ndarray, k_rope: np.ndarray,
                  u_k: np.ndarray, u_v: np.ndarray, scale: float,
                  key_weight: Optional[np.ndarray] = None, key_rinv: Optional[np.ndarray] = None):
    """One query row of one head, in the direct form.

    q_nope [d_nope]; q_rot [d_rope] (rotated at the query's true position);
    c [n, d_c] latents; k_rope [n, d_rope] rotary keys at their true positions;
    u_k [d_nope, d_c]; u_v [d_v, d_c].

    Expands k^C_t = U_K c_t and v_t = U_V c_t explicitly, scores
    s_t = scale * (q^C . k^C_t + q^R . k^R_t), softmaxes, and returns
    (o = sum_t a_t v_t, o_lat = sum_t a_t c_t, lse).  With QK-Norm the
    expanded content key is normalised first: k^C_t <- key_weight *
    k^C_t * key_rinv[t] (key_rinv: inverse RMS of row t's key over all heads)."""
    n = c.shape[0]
    d_v, d_c = u_v.shape
    if n == 0:
        return np.zeros(d_v), np.zeros(d_c), NEG_INF
    k_c = expand(u_k, c)                   # [n, d_nope]
    if key_weight is not None:
        k_c = k_c * np.asarray(key_weight, np.float64)[None, :]
    if key_rinv is not None:
        k_c = k_c * np.asarray(key_rinv, np.float64)[:, None]
    s = scale * (k_c @ np.asarray(q_nope, np.float64) + np.asarray(k_rope, np.float64) @ q_rot)
    a, lse = softmax_lse(s)
    v = expand(u_v, c)                     # [n, d_v]
    return a @ v, a @ np.asarray(c, np.float64), lse


def merge_lse(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge partial attention states of disjoint key sets by log-sum-exp.

    o_parts [n, d] are the normalised partial outputs, lse_parts [n] their
    log-sum-exps (-inf for an empty part).  The merged state is
    lse = ln sum_j exp(lse_j) and o = sum_j exp(lse_j - lse) o_j, which is the
    softmax over the union of the key sets (RedKnot-MLA abstract: the two
    paths are merged before one shared output projection)."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    live = np.isfinite(lse_parts)
    if not live.any():
        return np.zeros(o_parts.shape[1:]), NEG_INF
    m = lse_parts[live].max()
    w = np.where(live, np.exp(np.where(live, lse_parts, 0.0) - m), 0.0)
    tot = w.sum()
    lse = float(m + math.log(tot))
    o = (w[:, None] * np.where(live[:, None], o_parts, 0.0)).sum(axis=0) / tot
    return o, lse


# --------------------------------------------------------------------------
# QK-Norm (QK-Norm MLA page, abstract): RMSNorm after the projections
# --------------------------------------------------------------------------
@dataclass
class QKNorm:
    """Post-projection RMSNorm, RMSNorm(x) = g * x / sqrt(mean(x^2) + eps), of
    the content query and the content key.  The statistic runs over the whole
    projection of a token: the query over all heads' q_nope, the key over all
    heads' U_K c_t (the heads share one latent, one KV group).  g_q, g_k
    [H, d_nope].  The rotary parts are not normalised."""
    g_q: np.ndarray
    g_k: np.ndarray
    eps: float


def rms_inverse(x: np.ndarray, eps: float) -> float:
    """1 / sqrt(mean(x^2) + eps) over every entry of x."""
    x = np.asarray(x, np.float64)
    return 1.0 / math.sqrt(float(np.mean(x * x)) + eps)


def key_rms_inverse(w_uk: np.ndarray, c: np.ndarray, eps: float) -> np.ndarray:
    """Inverse RMS of each row's expanded content key over all heads:
    w_uk [H, d_nope, d_c], c [n, d_c] -> [n] (rows expanded in chunks)."""
    w = np.asarray(w_uk, np.float64)
    c = np.asarray(c, np.float64)
    out = np.empty(c.shape[0])
    for i in range(0, c.shape[0], 1024):
        k = np.einsum("hjd,nd->nhj", w, c[i:i + 1024])   # U_K[h] c_t, every head
        out[i:i + 1024] = 1.0 / np.sqrt(np.mean(k * k, axis=(1, 2)) + eps)
    return out


# --------------------------------------------------------------------------
# Whole decode step over KV segments
# --------------------------------------------------------------------------
@dataclass
class OracleSegment:
    """One KV segment as the oracle sees it.

    rows(b) -> [T_b, d_c + d_rope] array of stored rows [c_t | kr_t] of request b
    shift[b]: true position = stored position + shift[b]
    heads [head_begin, head_begin + head_count) read this segment."""
    rows: Callable[[int], np.ndarray]
    shift: Sequence[int]
    head_begin: int
    head_count: int
    causal: bool


def direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv, segments: List[OracleSegment],
                      scale: float, rope_base: float, s_q: int,
                      requests: Optional[Sequence[int]] = None,
                      heads: Optional[Sequence[int]] = None,
                      qk_norm: Optional[QKNorm] = None):
    """Direct-form decode for query tokens t = b * s_q + s and heads h.

    Returns (o [n_tok, H, d_v], o_lat [n_tok, H, d_c], lse [n_tok, H]); entries
    for (request, head) pairs not asked for are NaN.  For each head the keys of
    every segment whose head range holds it are concatenated into one softmax
    (step order: pick segments, expand content keys, move rotary keys to their
    true positions, rotate the query at its true position, score, softmax,
    expand values, weight).  With qk_norm the expanded content query and key
    are RMS-normalised before the score."""
    q_nope = np.asarray(q_nope, np.float64)
    q_pe = np.asarray(q_pe, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_tok, H, _ = q_nope.shape
    B = n_tok // s_q
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    requests = range(B) if requests is None else requests
    heads = range(H) if heads is None else heads
    o = np.full((n_tok, H, d_v), np.nan)
    o_lat = np.full((n_tok, H, d_c), np.nan)
    lse = np.full((n_tok, H), np.nan)
    for b in requests:
        seg_rows = []
        for seg in segments:
            r = np.asarray(seg.rows(b), np.float64)
            c = r[:, :d_c]
            kr_true = rope_rotate(r[:, d_c:], int(seg.shift[b]), rope_base)  # key-side relocation
            kinv = key_rms_inverse(w_uk, c, qk_norm.eps) if qk_norm is not None else None
            seg_rows.append((c, kr_true, kinv))
        for s in range(s_q):
            t = b * s_q + s
            qinv = rms_inverse(q_nope[t], qk_norm.eps) if qk_norm is not None else None
            for h in heads:
                cs, ks, kis = [], [], []
                for seg, (c, kr, kinv) in zip(segments, seg_rows):
                    if not (seg.head_begin <= h < seg.head_begin + seg.head_count):
                        continue
                    n = c.shape[0]
                    vis = n - s_q + s + 1 if seg.causal else n
                    vis = max(0, min(n, vis))
                    cs.append(c[:vis])
                    ks.append(kr[:vis])
                    if kinv is not None:
                        kis.append(kinv[:vis])
                c_all = np.concatenate(cs) if cs else np.zeros((0, d_c))
                k_all = np.concatenate(ks) if ks else np.zeros((0, q_pe.shape[2]))
                q_rot = rope_rotate(q_pe[t, h], int(q_pos[t]), rope_base)
                if qk_norm is None:
                    o[t, h], o_lat[t, h], lse[t, h] = attend_direct(
                        q_nope[t, h], q_rot, c_all, k_all, w_uk[h], w_uv[h], scale)
                else:
                    q_c = np.asarray(qk_norm.g_q, np.float64)[h] * q_nope[t, h] * qinv
                    k_inv = np.concatenate(kis) if kis else np.zeros(0)
                    o[t, h], o_lat[t, h], lse[t, h] = attend_direct(
                        q_c, q_rot, c_all, k_all, w_uk[h], w_uv[h], scale,
                        key_weight=np.asarray(qk_norm.g_k, np.float64)[h], key_rinv=k_inv)
    return o, o_lat, lse


def cache_bytes(n_layers: int, batch: int, tokens: int, d_c: int, d_r: int, bytes_per: int) -> int:
    """Stored MLA cache size: one latent (d_c) and one rotary key (d_r) per
    layer-token, no factor of two on the latent ("Count the Cache That Is
    Actually Stored")."""
    return n_layers * batch * tokens * (d_c + d_r) * bytes_per


def mha_cache_bytes(n_layers: int, batch: int, tokens: int, n_heads: int, d_k: int, d_v: int,
                    bytes_per: int) -> int:
    """Ordinary multi-head cache: a key and a value per head per layer-token
    ("Start With What Ordinary Attention Saves")."""
    return n_layers * batch * tokens * n_heads * (d_k + d_v) * bytes_per
