"""Planted mistakes in the oracle must each break at least one pin (CPU only).

Each mutant rewrites one expression of the oracle's source (a dropped term, a
wrong sign, index, axis or operand) into a fresh module; the pins in
``oracle_pins`` are then run against it and at least one must fail.  This
shows the pins constrain every step of the oracle, not just its shape.
"""
import importlib.util
import os
import types

import pytest

from oracle_pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "monarch_oracle.py")

MUTANTS = {
    "drop_entropy_term": ("+ h_r[g].T[:, None, :]", "+ 0.0"),
    "entropy_sign": ("h_r = entropy(R, axis=-1)", "h_r = -entropy(R, axis=-1)"),
    "drop_beta": ("q_hat[g] = qh.transpose(1, 0, 2)", "q_hat[g] = q_til.transpose(1, 0, 2)"),
    "drop_scale_r": ("logits = s * (q_hat[g] @ kb.transpose(0, 2, 1))",
                     "logits = (q_hat[g] @ kb.transpose(0, 2, 1))"),
    "drop_scale_l": ("logits[:, lo:hi, :] = s * (q_cols", "logits[:, lo:hi, :] = (q_cols"),
    "l_softmax_axis": ("return softmax(logits, axis=-1), logits",
                       "return softmax(logits, axis=1), logits"),
    "r_softmax_axis": ("R[g] = softmax(logits, axis=-1)", "R[g] = softmax(logits, axis=1)"),
    "ktil_R_transposed": ('np.einsum("gcap,cpd->gcad", R, kb)', 'np.einsum("gcpa,cpd->gcad", R, kb)'),
    "apply_R_transposed": ("U = R[g] @ vb", "U = R[g].transpose(0, 2, 1) @ vb"),
    "apply_L_transposed": ("y_cols = L[:, lo:hi, :] @ U.transpose(1, 0, 2)",
                           "y_cols = L.transpose(0, 2, 1)[:, lo:hi, :] @ U.transpose(1, 0, 2)"),
    "r_step_whole_column": ("Lg = L[:, lo:hi, :]", "Lg = L[:, :, :] * 0 + L[:, :, :]; q_cols = qb.transpose(1, 0, 2)"),
    "r_step_keys_as_queries": ("q_cols = qb[lo:hi].transpose(1, 0, 2)             # [a2, a1 in g, d]\n        mass",
                               "q_cols = kb[lo:hi].transpose(1, 0, 2)\n        mass"),
    "l_step_tile0_keys": ("k_cols = k_til[g].transpose(1, 0, 2)", "k_cols = k_til[0].transpose(1, 0, 2)"),
    "apply_tile0_R": ("U = R[g] @ vb", "U = R[0] @ vb"),
    "init_not_uniform": ("return np.full((t, b1, b2, b2), 1.0 / b2)",
                         "return np.broadcast_to(np.eye(b2), (t, b1, b2, b2)).copy()"),
    "tile_bounds_drop_last_row": ("return [(g * b1) // t for g in range(t + 1)]",
                                  "return [(g * b1) // t for g in range(t)] + [b1 - 1]"),
    "tile_bounds_uneven": ("return [(g * b1) // t for g in range(t + 1)]",
                           "return [0] + [min(b1, g * (b1 // t + 1)) for g in range(1, t)] + [b1]"),
    "kbar_from_values": ("L, _ = l_step(qb, kb, R, bounds, s)", "L, _ = l_step(qb, vb, R, bounds, s)"),
    "apply_values_are_keys": ("y = apply_factors(L, R, vb, bounds)", "y = apply_factors(L, R, kb, bounds)"),
    "dense_M_wrong_tile": ("Rg = R[g_of[a1]]", "Rg = R[0]"),
    "kv_tiles_over_key_blocks": ("bounds = tile_bounds(b1q, tiles)", "bounds = tile_bounds(b1, tiles)"),
    "kv_apply_rows_from_keys": ("y = np.empty((L.shape[1], b2, d))", "y = np.zeros((vb.shape[0], b2, d))"),
    "adaptive_gain_not_per_token": ("(F[-1] - F[-2]) / Nq <= tol", "(F[-1] - F[-2]) <= tol"),
    "adaptive_stops_after_one": ("(it >= 2 and (F[-1] - F[-2]) / Nq <= tol)", "(it >= 1 and (F[-1] - F[-2 if it > 1 else -1]) / Nq <= tol)"),
    "adaptive_objective_without_max": ("F.append(float(np.sum(m[..., 0] + np.log(", "F.append(float(np.sum(0 * m[..., 0] + np.log("),
    "beta_zero_tile_mean": ("qh = np.where((mass > 0)[:, :, None], q_til / safe[:, :, None], 0.0)",
                            "qh = np.where((mass > 0)[:, :, None], q_til / safe[:, :, None], "
                            "q_cols.mean(axis=1)[:, None, :])"),
    "beta_zero_first_query": ("qh = np.where((mass > 0)[:, :, None], q_til / safe[:, :, None], 0.0)",
                              "qh = np.where((mass > 0)[:, :, None], q_til / safe[:, :, None], "
                              "q_cols[:, :1, :])"),
    "stale_L_in_apply": ("        R, _, _ = r_step(qb, kb, L, bounds, s)\n        history",
                         "        R, _, _ = r_step(qb, kb, L, bounds, s)\n        L = L[:, ::-1, :]\n        history"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), SRC + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # an assertion, or a crash the mistake causes
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
