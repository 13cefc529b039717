"""The oracle's pins have teeth: plant one mistake at a time in a scratch copy
of the oracle's C source (on the CPU, never on a GPU) and check that the pins
which do not compare the oracle's two recurrence forms with each other fail.

Mistakes planted: the previous-token term skipping the step's rotation/decay,
the rotation direction, the sign of C's or B's imaginary part, trapezoid
weights swapped, rank columns mixed, the D term dropped, a stale previous
token, a sigmoid instead of a SiLU gate, an L2 instead of an RMS norm, the
norm's eps added outside the root, every head taking head 0's bias; and in
the gradient: the rotation's transpose taken the wrong way, the angle
derivative's sign, the previous-token weight dropped from its gradient, the
norm's Jacobian reduced to its diagonal, the gate's derivative without its
input factor, and the decay's share of the step's gradient dropped; in the variants, a
per-token decay rate halved, the fixed trapezoid weight ignored and heads
mapped to the wrong shared angle row; in the chunked SSD form, the carried
state's fold taking another token's weight, its final state rotated the wrong
way and the in-chunk decay missing its first factor."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "prev_not_rotated": ("hc[k * P + p] = z[k] * (hc[k * P + p] + delta * prev) + gamma * cur;",
                         "hc[k * P + p] = z[k] * hc[k * P + p] + delta * prev + gamma * cur;"),
    "rotation_sign": ("z[k] = decay * (cos(ang) + I * sin(ang));", "z[k] = decay * (cos(ang) - I * sin(ang));"),
    "c_imag_sign": ("cc[k * R + j] = row2[2 * k] - I * row2[2 * k + 1];",
                    "cc[k * R + j] = row2[2 * k] + I * row2[2 * k + 1];"),
    "b_imag_sign": ("bc[k * R + j] = row[2 * k] + I * row[2 * k + 1];",
                    "bc[k * R + j] = row[2 * k] - I * row[2 * k + 1];"),
    "weights_swapped": ("const double delta = (1.0 - lam) * dt, gamma = lam * dt;",
                        "const double gamma = (1.0 - lam) * dt, delta = lam * dt;"),
    "rank_mixed": ("cur += bc[k * R + j] * xc[p * R + j];", "cur += bc[k * R + j] * xc[p * R + 0];"),
    "no_skip_term": ("yt[i * P + p] = gate(a, creal(acc) + Dh * xc[p * R + i], ox + i * P + p);",
                     "yt[i * P + p] = gate(a, creal(acc), ox + i * P + p);"),
    "gate_sigmoid_only": ("return y * v / (1.0 + exp(-v));", "return y / (1.0 + exp(-v));"),
    "norm_without_mean": ("1.0 / sqrt(ss / N + a->bc_eps);\n        for (int n = 0; n < N; n++) out[n] *= inv;",
                          "1.0 / sqrt(ss + a->bc_eps);\n        for (int n = 0; n < N; n++) out[n] *= inv;"),
    "eps_outside_root": ("1.0 / sqrt(ss / N + a->bc_eps);\n        for (int n = 0; n < N; n++) out[n] *= inv;",
                         "1.0 / (sqrt(ss / N) + a->bc_eps);\n        for (int n = 0; n < N; n++) out[n] *= inv;"),
    "bias_of_head_zero": ("out[n] += bias[(int64_t)h * N + n];", "out[n] += bias[n];"),
    "grad_rotation_transposed": ("V[(2 * k) * P + p] = alpha * (c * g0 + sn * g1);",
                                 "V[(2 * k) * P + p] = alpha * (c * g0 - sn * g1);"),
    "grad_angle_sign": ("acc += g0 * (-sn * u0 - c * u1) + g1 * (c * u0 - sn * u1);",
                        "acc += g0 * (sn * u0 - c * u1) + g1 * (c * u0 - sn * u1);"),
    "grad_prev_weight_dropped": ("dBp[j * N + n] += delta * V[n * P + p] * Xp[j * P + p];",
                                 "dBp[j * N + n] += V[n * P + p] * Xp[j * P + p];"),
    "grad_norm_jacobian_dropped": ("graw[m] += gout[m] * inv - dot * inv * inv * inv * v[m] / N;",
                                   "graw[m] += gout[m] * inv;"),
    "grad_gate_without_input": ("dy0[i * P + p] = d * v * sg;", "dy0[i * P + p] = d * sg;"),
    "grad_decay_chain_dropped": ("double ddt = Ah * alpha * dalpha + (1.0 - lam) * ddelta + lam * dgamma;",
                                 "double ddt = (1.0 - lam) * ddelta + lam * dgamma;"),
    "per_token_decay_halved": ("return a->A_tok ? ld(a->A_tok, a->in_dtype, i) : a->A[h];",
                               "return a->A_tok ? 0.5 * ld(a->A_tok, a->in_dtype, i) : a->A[h];"),
    "fixed_lambda_ignored": ("return a->lam ? ld(a->lam, a->in_dtype, i) : a->lam_fixed;",
                             "return a->lam ? ld(a->lam, a->in_dtype, i) : 0.5;"),
    "angle_group_of_head": ("return (t * Gth + h / (a->H / Gth)) * K + k;", "return (t * Gth + h % Gth) * K + k;"),
    # the chunked SSD form: the carried state's fold taking the chunk's second token's weight, the
    # final state rotated the wrong way, the in-chunk decay missing its first factor
    "chunked_fold_wrong_token": ("Hs[n * P + p] += delta[0] * acc;", "Hs[n * P + p] += delta[nq > 1 ? 1 : 0] * acc;"),
    "chunked_state_rotation_sign": ("Hs[(2 * k) * P + p] = c * u - sn * v;\n                Hs[(2 * k + 1) * P + p] = sn * u + c * v;",
                                    "Hs[(2 * k) * P + p] = c * u + sn * v;\n                Hs[(2 * k + 1) * P + p] = -sn * u + c * v;"),
    "chunked_decay_first_factor": ("for (int k = 0; k <= t; k++) decay *= alpha[k];", "for (int k = 1; k <= t; k++) decay *= alpha[k];"),
    "stale_previous": ("memcpy(bp, bc, (size_t)K * R * sizeof *bp);\n        memcpy(xp, xc, (size_t)P * R * sizeof *xp);\n",
                       ""),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "m3_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor moved; update the anchor"
    work = tmp_path / "tree"
    os.makedirs(work)
    shutil.copytree(os.path.join(ROOT, "oracle"), work / "oracle", ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), work / "tests", ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "state_space_sequence_mamba3_amd"), work / "state_space_sequence_mamba3_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "_build"))
    (work / "oracle" / "m3_oracle.c").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "-k", "not rotated_frame"],
                       cwd=work, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and " failed" in r.stdout, r.stdout[-2000:]
