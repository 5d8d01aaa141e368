"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant rewrites one expression of the oracle's source (a dropped term,
a wrong sign, index or divisor, a transposed operand, a lost precision) and
is loaded as a separate module; the real oracle is never touched.
"""

import os
import types

import pytest

import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "coda_oracle.py")

MUTANTS = [
    ("gemm_in_fp32", "return _f(a) @ _f(b)", "return (np.asarray(a, np.float32) @ np.asarray(b, np.float32)).astype(F64)"),
    ("residual_sign", "return gemm(x, w0) + _f(z)", "return gemm(x, w0) - _f(z)"),
    ("sumsq_on_scaled", "return u, u * _f(gamma)[None, :], row_sumsq(u)", "return u, u * _f(gamma)[None, :], row_sumsq(u * _f(gamma)[None, :])"),
    ("eps_outside_sqrt", "return 1.0 / np.sqrt(_f(sumsq) / d + eps)", "return 1.0 / (np.sqrt(_f(sumsq) / d) + eps)"),
    ("rms_divisor", "return 1.0 / np.sqrt(_f(sumsq) / d + eps)", "return 1.0 / np.sqrt(_f(sumsq) / (d - 1) + eps)"),
    ("rmsnorm_no_gamma", "return (r[:, None] * u) * _f(gamma)[None, :], r", "return (r[:, None] * u), r"),
    ("rmsnorm_rsqrt_of_sum", "r = 1.0 / np.sqrt(np.mean(u * u, axis=1) + eps)\n    return", "r = 1.0 / np.sqrt(np.sum(u * u, axis=1) + eps)\n    return"),
    ("rope_sign", "y[:, 0:n_rope:2] = a * cs - b * sn", "y[:, 0:n_rope:2] = a * cs + b * sn"),
    ("rope_no_head_reset", "k = (c % head_dim) // 2", "k = c // 2"),
    ("rope_exponent", "-2.0 * k / head_dim", "-1.0 * k / head_dim"),
    ("rope_pair_swap", "b = t[:, 1:n_rope:2]\n    y[", "b = t[:, 0:n_rope:2]\n    y["),
    ("swiglu_gate_up_swapped", "g = pre[:, 0::2]\n    v = pre[:, 1::2]\n    return", "g = pre[:, 1::2]\n    v = pre[:, 0::2]\n    return"),
    ("swiglu_bwd_term", "out[:, 0::2] = da * v * s * (1.0 + g * (1.0 - s))", "out[:, 0::2] = da * v * s * (1.0 + g * s)"),
    ("swiglu_bwd_dv", "out[:, 1::2] = da * g * s", "out[:, 1::2] = da * s"),
    ("ce_sign", "loss = lse - tgt", "loss = tgt - lse"),
    ("ce_mean", "return lse, loss, float(np.mean(loss))", "return lse, loss, float(np.sum(loss))"),
    ("ce_no_max_add", "return m + np.log(np.sum(np.exp(l - m[:, None]), axis=1))", "return np.log(np.sum(np.exp(l - m[:, None]), axis=1))"),
    ("ce_bwd_onehot_sign", "p[np.arange(l.shape[0]), labels] -= 1.0", "p[np.arange(l.shape[0]), labels] += 1.0"),
    ("ce_bwd_dW_scaled", "return gemm(D, w.T), gemm(h.T, D), D", "return gemm(D, w.T), gemm(h.T, D) * 0.5, D"),
    ("rmsnorm_bwd_no_mean_term", "du = r[:, None] * gn - (r ** 3)[:, None] * u * np.mean(gn * u, axis=1)[:, None]", "du = r[:, None] * gn"),
    ("rmsnorm_bwd_r_power", "du = r[:, None] * gn - (r ** 3)[:, None]", "du = r[:, None] * gn - (r ** 2)[:, None]"),
    ("rmsnorm_bwd_dgamma_no_r", "dgamma = np.sum(dn2 * (r[:, None] * u), axis=0)", "dgamma = np.sum(dn2 * u, axis=0)"),
    ("s_divisor", "s = np.sum(dn2 * n2, axis=1) / d", "s = np.sum(dn2 * n2, axis=1)"),
    ("block_fwd_no_residual", "u2 = gemm(a1, p[\"Wd1\"]) + u1", "u2 = gemm(a1, p[\"Wd1\"])"),
    ("block_bwd_skip_grad", "eps, dres=g[\"du2\"])", "eps, dres=dOut)"),
    ("block_bwd_wgrad_operand", "g[\"dWgu2\"] = gemm(f[\"n2_2\"].T, g[\"dpre2\"])", "g[\"dWgu2\"] = gemm(f[\"u2\"].T, g[\"dpre2\"])"),
    ("mlp_bwd_no_residual", "dX = gemm(dpre, _f(wgu).T) + dY", "dX = gemm(dpre, _f(wgu).T)"),
    ("ln_no_centering", "cu = u - mu[:, None]", "cu = u"),
    ("ln_unbiased_var", "r = 1.0 / np.sqrt(np.mean(cu * cu, axis=1) + eps)",
     "r = 1.0 / np.sqrt(np.sum(cu * cu, axis=1) / (u.shape[1] - 1) + eps)"),
    ("ln_eps_outside_sqrt", "r = 1.0 / np.sqrt(np.mean(cu * cu, axis=1) + eps)",
     "r = 1.0 / (np.sqrt(np.mean(cu * cu, axis=1)) + eps)"),
    ("ln_no_beta", "* _f(gamma)[None, :] + _f(beta)[None, :], mu, r", "* _f(gamma)[None, :], mu, r"),
    ("ln_beta_before_gamma", "return (r[:, None] * cu) * _f(gamma)[None, :] + _f(beta)[None, :], mu, r",
     "return (r[:, None] * cu + _f(beta)[None, :]) * _f(gamma)[None, :], mu, r"),
    ("ln_bwd_no_mean_term", "du = r[:, None] * (gn - a[:, None] - xhat * s[:, None])",
     "du = r[:, None] * (gn - xhat * s[:, None])"),
    ("ln_bwd_no_s_term", "du = r[:, None] * (gn - a[:, None] - xhat * s[:, None])",
     "du = r[:, None] * (gn - a[:, None])"),
    ("ln_bwd_uncentered", "centered = u - mu[:, None]", "centered = u"),
    ("ln_bwd_dgamma_no_r", "dgamma = np.sum(dn * xhat, axis=0)", "dgamma = np.sum(dn * centered, axis=0)"),
    ("ln_bwd_dbeta_gamma", "dbeta = np.sum(dn, axis=0)", "dbeta = np.sum(dn * gamma[None, :], axis=0)"),
    ("ln_block_wgrad_operand", "g[\"dWgu1\"] = gemm(f[\"n_1\"].T, g[\"dpre1\"])",
     "g[\"dWgu1\"] = gemm(f[\"u1\"].T, g[\"dpre1\"])"),
    ("ln_block_fwd_no_residual", "u2 = u1 + gemm(a1, p[\"Wd1\"])", "u2 = gemm(a1, p[\"Wd1\"])"),
    ("ln_block_fwd_no_beta2", "layernorm(u2, p[\"gamma2\"], p[\"beta2\"], eps)",
     "layernorm(u2, p[\"gamma2\"], 0.0 * p[\"beta2\"], eps)"),
]


def _load_mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # AssertionError or a shape error both count as caught
            caught.append(check.__name__)
    assert caught, f"planted mistake {name} passed every pin"
