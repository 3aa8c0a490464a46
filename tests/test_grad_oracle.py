"""The gradient oracle against facts it does not compute itself, and planted
mistakes in it that those facts must catch (CPU only)."""
import os
import types

import pytest

import oracle.monarch_grad as grad_oracle
from grad_pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "monarch_grad.py")

MUTANTS = {
    "dL_apply_missing": ("dL[:, lo:hi, :] = dy_cols @ Ug.transpose(0, 2, 1)",
                         "dL[:, lo:hi, :] = 0.0 * (dy_cols @ Ug.transpose(0, 2, 1))"),
    "dU_unweighted": ("dU = (Lg.transpose(0, 2, 1) @ dy_cols)", "dU = (np.ones_like(Lg).transpose(0, 2, 1) @ dy_cols)"),
    "dv_R_not_transposed": ("dvb += Rs[T][g].transpose(0, 2, 1) @ dU", "dvb += Rs[T][g] @ dU"),
    "dz_no_centering": ("dz = R[g] * (dR[g] - np.sum(R[g] * dR[g], axis=-1, keepdims=True))", "dz = R[g] * dR[g]"),
    "dqhat_no_scale": ("dq_hat = s * (dz @ kb)", "dq_hat = (dz @ kb)"),
    "dk_r_missing": ("dkb += s * (dz.transpose(0, 2, 1) @ q_hat[g])", "pass"),
    "G_no_beta": ("dq_hat / np.where(mass > 0, mass, 1.0)[:, :, None]", "dq_hat"),
    "dL_agg_no_qhat_term": ("- np.sum(Gc * qh_c, axis=-1)[:, None, :]", "- 0.0"),
    "dL_agg_sign": ("dL[:, lo:hi, :] += q_cols @ Gc.transpose(0, 2, 1)", "dL[:, lo:hi, :] -= q_cols @ Gc.transpose(0, 2, 1)"),
    "dq_agg_missing": ("dqb[lo:hi] += (Lg @ Gc).transpose(1, 0, 2)", "pass"),
    "dl_no_centering": ("dl = L * (dL - np.sum(L * dL, axis=-1, keepdims=True))", "dl = L * dL"),
    "dq_l_missing": ("dqb[lo:hi] += (s * (dlg @ k_cols)).transpose(1, 0, 2)", "pass"),
    "dkbar_not_mean": ("dkb += dk_til.sum(axis=(0, 2))[:, None, :] / b2", "dkb += dk_til.sum(axis=(0, 2))[:, None, :]"),
    "dktil_wrong_operand": ("dk_til[g] = (s * (dlg.transpose(0, 2, 1) @ q_perm[:, lo:hi, :]))",
                            "dk_til[g] = (s * (dlg.transpose(0, 2, 1) @ q_perm[:, hi - (hi - lo):hi, :][:, ::-1, :]))"),
    # several iterations
    "entropy_grad_sign": ("- dh[..., None] * (logR + 1.0)", "+ dh[..., None] * (logR + 1.0)"),
    "entropy_grad_missing": ("- dh[..., None] * (logR + 1.0)", "- 0.0 * dh[..., None]"),
    "ktil_grad_to_k_missing": ('dkb += np.einsum("gcap,gcad->cpd", Rp, dk_til)', "pass"),
    "ktil_grad_R_transposed": ('dkb += np.einsum("gcap,gcad->cpd", Rp, dk_til)', 'dkb += np.einsum("gcpa,gcad->cpd", Rp, dk_til)'),
    "stale_dL_between_iterations": ("            dL = np.zeros_like(Ls[i - 1])", "            dL = dL * 1.0"),
    "earlier_iterations_use_last_L": ("        R, L, q_hat, beta = Rs[i], Ls[i], qhats[i], betas[i]",
                                      "        R, L, q_hat, beta = Rs[i], Ls[T], qhats[i], betas[i]"),
    "tile0_U": ("Ug = U[g].transpose(1, 0, 2)", "Ug = U[0].transpose(1, 0, 2)"),
    # a chunk of query frames against cached keys
    "chunk_tiles_over_key_blocks": ("bounds = tile_bounds(b1q, tiles)", "bounds = tile_bounds(b1, tiles)"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle.monarch_grad_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), SRC + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(grad_oracle)


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
