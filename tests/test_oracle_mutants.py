"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (a dropped term, a wrong sign, index or operand)."""
import sys
import types

import pytest

import oracle.mla_direct as O
from oracle_pins import ALL_PINS

SRC = open(O.__file__).read()

MUTANTS = {
    "wo_wrong_block": ("out += x[:, h, :] @ w[:, h * d_v:(h + 1) * d_v].T", "out += x[:, h, :] @ w[:, 0:d_v].T"),
    "wo_untransposed_block": ("out += x[:, h, :] @ w[:, h * d_v:(h + 1) * d_v].T",
                              "out += (w[:, h * d_v:(h + 1) * d_v] @ x[:, h, :].T).T[:, ::-1]"),
    "wo_last_head_only": ("out += x[:, h, :] @ w[:, h * d_v:(h + 1) * d_v].T",
                          "out = x[:, h, :] @ w[:, h * d_v:(h + 1) * d_v].T"),
    "fold_transposed_uv": ("return np.stack([w[:, h * d_v:(h + 1) * d_v] @ u[h] for h in range(H)])",
                           "return np.stack([w[:, h * d_v:(h + 1) * d_v] @ u[H - 1 - h] for h in range(H)])"),
    "rope_sign": ("out[..., 0::2] = x0 * cos - x1 * sin", "out[..., 0::2] = x0 * cos + x1 * sin"),
    "rope_freq": ("return base ** (-2.0 * i / d_rope)", "return base ** (-1.0 * i / d_rope)"),
    "rope_pairs_halves": ("x0, x1 = x[..., 0::2], x[..., 1::2]",
                          "x0, x1 = x[..., : d // 2], x[..., d // 2:]"),
    "relocate_sign": ("rel = np.asarray(pos, dtype=np.int64) - np.asarray(shift, dtype=np.int64)",
                      "rel = np.asarray(pos, dtype=np.int64) + np.asarray(shift, dtype=np.int64)"),
    "drop_rope_term": ("s = scale * (k_c @ np.asarray(q_nope, np.float64) + np.asarray(k_rope, np.float64) @ q_rot)",
                       "s = scale * (k_c @ np.asarray(q_nope, np.float64))"),
    "scale_content_only": ("s = scale * (k_c @ np.asarray(q_nope, np.float64) + np.asarray(k_rope, np.float64) @ q_rot)",
                           "s = scale * (k_c @ np.asarray(q_nope, np.float64)) + np.asarray(k_rope, np.float64) @ q_rot"),
    "lse_log2": ("return e / tot, float(m + math.log(tot))", "return e / tot, float(m + math.log2(tot))"),
    "lse_no_max": ("return e / tot, float(m + math.log(tot))", "return e / tot, float(math.log(tot))"),
    "value_from_keys": ("v = expand(u_v, c)                     # [n, d_v]",
                        "v = expand(u_k, c)[:, : u_v.shape[0]]"),
    "o_lat_unweighted": ("return a @ v, a @ np.asarray(c, np.float64), lse",
                         "return a @ v, np.asarray(c, np.float64).mean(axis=0), lse"),
    "absorb_wrong_head": ("out[:, h, :] = q[:, h, :] @ w[h]\n", "out[:, h, :] = q[:, h, :] @ w[-1 - h]\n"),
    "output_wrong_head": ("out[:, h, :] = o[:, h, :] @ w[h].T", "out[:, h, :] = o[:, h, :] @ w[0].T"),
    "causal_off_by_one": ("vis = n - s_q + s + 1 if seg.causal else n", "vis = n - s_q + s if seg.causal else n"),
    "shift_ignored": ("kr_true = rope_rotate(r[:, d_c:], int(seg.shift[b]), rope_base)",
                      "kr_true = r[:, d_c:]"),
    "head_range_ignored": ("if not (seg.head_begin <= h < seg.head_begin + seg.head_count):",
                           "if False:"),
    "merge_unnormalised": ("o = (w[:, None] * np.where(live[:, None], o_parts, 0.0)).sum(axis=0) / tot",
                           "o = (w[:, None] * np.where(live[:, None], o_parts, 0.0)).sum(axis=0)"),
    "merge_plain_sum_lse": ("lse = float(m + math.log(tot))", "lse = float(lse_parts[live].sum())"),
    "cache_factor_two": ("return n_layers * batch * tokens * (d_c + d_r) * bytes_per",
                         "return n_layers * batch * tokens * (2 * d_c + d_r) * bytes_per"),
    "qknorm_key_rms_one_head": ("out[i:i + 1024] = 1.0 / np.sqrt(np.mean(k * k, axis=(1, 2)) + eps)",
                                "out[i:i + 1024] = 1.0 / np.sqrt(np.mean(k[:, :1] * k[:, :1], axis=(1, 2)) + eps)"),
    "qknorm_eps_outside_sqrt": ("out[i:i + 1024] = 1.0 / np.sqrt(np.mean(k * k, axis=(1, 2)) + eps)",
                                "out[i:i + 1024] = 1.0 / (np.sqrt(np.mean(k * k, axis=(1, 2))) + eps)"),
    "qknorm_key_weight_dropped": ("k_c = k_c * np.asarray(key_weight, np.float64)[None, :]", "k_c = k_c"),
    "qknorm_query_rms_one_head": ("qinv = rms_inverse(q_nope[t], qk_norm.eps) if qk_norm is not None else None",
                                  "qinv = rms_inverse(q_nope[t, 0], qk_norm.eps) if qk_norm is not None else None"),
    "qknorm_query_weight_from_key": ("q_c = np.asarray(qk_norm.g_q, np.float64)[h] * q_nope[t, h] * qinv",
                                     "q_c = np.asarray(qk_norm.g_k, np.float64)[h] * q_nope[t, h] * qinv"),
    "query_rot_wrong_pos": ("q_rot = rope_rotate(q_pe[t, h], int(q_pos[t]), rope_base)",
                            "q_rot = rope_rotate(q_pe[t, h], int(q_pos[t]) - 1, rope_base)"),
}


def _mutant(old, new):
    assert old in SRC, f"mutation site vanished: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = O.__file__
    sys.modules["oracle_mutant"] = mod  # dataclasses look their module up
    try:
        exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {name} passed every pin"
