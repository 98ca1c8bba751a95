"""Plants plausible mistakes in copies of the oracle source (on the CPU) and
checks that every mutant fails at least one pin. This shows the pins would catch
a dropped term, a wrong sign, a wrong index or a transposed operand."""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC_DIR = os.path.dirname(os.path.abspath(oracle.__file__))

# (name, exact text in ssm_oracle.c, replacement)
MUTANTS = [
    ("decay_sign", "exp(delta * a[n]) * h[n]", "exp(-delta * a[n]) * h[n]"),
    ("euler_decay", "exp(delta * a[n]) * h[n]", "(1.0 + delta * a[n]) * h[n]"),
    ("drop_delta_in_input", "(delta * x_t) * B_t[n]", "x_t * B_t[n]"),
    ("input_wrong_state_index", "(delta * x_t) * B_t[n]", "(delta * x_t) * B_t[0]"),
    ("readout_uses_B", "s += C_t[n] * h[n];", "s += B_t[n] * h[n];"),
    ("skip_drops_x", "s += (*D_d) * x_t;", "s += (*D_d);"),
    ("gate_is_z", "s *= ssm_oracle_silu(*z_t);", "s *= *z_t;"),
    ("bias_dropped", "double v = delta_raw_t + (bias_d ? *bias_d : 0.0);",
     "double v = delta_raw_t;"),
    ("softplus_pos_branch", "return v + log1p(exp(-v));", "return log1p(exp(-v));"),
    ("softplus_is_exp", "return log1p(exp(v));", "return exp(v);"),
    ("silu_neg_branch", "sig = e / (1.0 + e);", "sig = 1.0 / (1.0 + e);"),
    ("B_time_off_by_one", "const double* Bt = j->B + (b * L + t) * N;",
     "const double* Bt = j->B + (b * L + (t > 0 ? t - 1 : 0)) * N;"),
    ("A_indexed_by_batch", "const double* a = j->A + d * N;", "const double* a = j->A + b * N;"),
    ("h0_ignored", "h[n] = j->h0 ? j->h0[r * N + n] : 0.0;", "h[n] = 0.0;"),
    ("z_first_token_only", "const double* zt = j->z ? j->z + r * L + t : NULL;",
     "const double* zt = j->z ? j->z + r * L : NULL;"),
    ("step_B_by_channel", "A + d * dstate, B + b * dstate, C + b * dstate,",
     "A + d * dstate, B + d * dstate, C + b * dstate,"),
    ("readout_before_update_skip", "    /* skip term D * x, then the gate silu(z) */\n    if (D_d)",
     "    /* skip term D * x, then the gate silu(z) */\n    if (0)"),
]


# the same, in the gradient file
BWD_MUTANTS = [
    ("bwd_decay_of_same_token", "G[n] = Gc[n] + dq * Ct[n];",
     "G[n] = Gc[n] * a[t * N + n] + dq * Ct[n];"),
    ("bwd_carry_skips_decay", "Gc[n] = a[t * N + n] * G[n];", "Gc[n] = G[n];"),
    ("bwd_dC_uses_prev_state", "j->dC[(b * L + t) * N + n] += dq * H[(t + 1) * N + n];",
     "j->dC[(b * L + t) * N + n] += dq * H[t * N + n];"),
    ("bwd_dB_drops_delta", "j->dB[(b * L + t) * N + n] += G[n] * (dl[t] * xr[t]);",
     "j->dB[(b * L + t) * N + n] += G[n] * xr[t];"),
    ("bwd_no_softplus_grad", "j->ddelta[r * L + t] = ddel * sg[t];",
     "j->ddelta[r * L + t] = ddel;"),
    ("bwd_dA_drops_delta", "j->dA[d * N + n] += gh * dl[t];", "j->dA[d * N + n] += gh;"),
    ("bwd_dz_drops_q", "j->dz[r * L + t] = dyt * q[t] * (sz * (1.0 + zt * (1.0 - sz)));",
     "j->dz[r * L + t] = dyt * (sz * (1.0 + zt * (1.0 - sz)));"),
    ("bwd_dsilu_is_sigmoid", "j->dz[r * L + t] = dyt * q[t] * (sz * (1.0 + zt * (1.0 - sz)));",
     "j->dz[r * L + t] = dyt * q[t] * sz;"),
    ("bwd_dx_drops_skip", "j->dx[r * L + t] = j->D ? dq * j->D[d] : 0.0;",
     "j->dx[r * L + t] = 0.0;"),
    ("bwd_dx_drops_delta", "j->dx[r * L + t] += du * dl[t];", "j->dx[r * L + t] += du;"),
    ("bwd_ddelta_drops_input_path", "ddel += du * xr[t];", "ddel += 0.0 * xr[t];"),
    ("bwd_dh0_undecayed", "j->dh0[r * N + n] = Gc[n];", "j->dh0[r * N + n] = G[n];"),
    ("bwd_dh_final_ignored", "Gc[n] = j->dh_final ? j->dh_final[r * N + n] : 0.0;",
     "Gc[n] = 0.0;"),
]

SOURCES = ["ssm_oracle.c", "ssm_oracle_bwd.c"]


def _mutant(tmp_path, name, fname, old, new):
    src = open(os.path.join(SRC_DIR, fname)).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    d = tmp_path / name
    d.mkdir()
    shutil.copy(os.path.join(SRC_DIR, "ssm_oracle.h"), d / "ssm_oracle.h")
    for f in SOURCES:
        text = open(os.path.join(SRC_DIR, f)).read()
        (d / f).write_text(src.replace(old, new) if f == fname else text)
    so = d / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", *[str(d / f) for f in SOURCES], "-o", str(so), "-lm"],
                   check=True)
    return so


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_mutant_is_caught(tmp_path, name, old, new):
    orc = oracle.Oracle(str(_mutant(tmp_path, name, "ssm_oracle_bwd.c", old, new)))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    so = _mutant(tmp_path, name, "ssm_oracle.c", old, new)
    orc = oracle.Oracle(str(so))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# Mistakes planted in the Python compositions of oracle/__init__.py (the reverse
# scan and packed sequences are built there from the C scan).
PY_MUTANTS = [
    ("rev_B_not_reversed", "rB = f64(B)[:, ::-1]", "rB = f64(B)"),
    ("rev_C_not_reversed", "rC = f64(C)[:, ::-1]", "rC = f64(C)"),
    ("rev_z_not_reversed", "rz = None if z is None else f64(z)[:, :, ::-1]",
     "rz = None if z is None else f64(z)"),
    ("rev_output_not_reversed", "return np.ascontiguousarray(y[:, :, ::-1]), hf",
     "return np.ascontiguousarray(y), hf"),
    ("varlen_h0_of_previous_seq", "start = None if h0f is None else h0f[i][None]",
     "start = None if h0f is None else h0f[max(i - 1, 0)][None]"),
    ("varlen_state_carried_across", "start = None if h0f is None else h0f[i][None]",
     "start = hf[i - 1][None] if i > 0 else None"),
    ("varlen_empty_final_zero", "hf[i] = 0.0 if start is None else start[0]", "hf[i] = 0.0"),
    ("varlen_C_from_row_start", "Cf[None, a:b]", "Cf[None, 0:b - a]"),
    ("varlen_bwd_dh_final_of_next_seq", "dh_final=None if dhf is None else dhf[i][None]",
     "dh_final=None if dhf is None else dhf[min(i + 1, nseq - 1)][None]"),
    ("varlen_bwd_empty_dh0_zero", 'out["dh0"][i] = 0.0 if dhf is None else dhf[i]',
     'out["dh0"][i] = 0.0'),
    ("varlen_bwd_dA_not_summed", 'out["dA"] += g["dA"]', 'out["dA"] = g["dA"]'),
    ("varlen_bwd_dB_at_row_start", 'out["dB"][a:b] = g["dB"][0]', 'out["dB"][0:b - a] = g["dB"][0]'),
    ("varlen_bwd_B_from_row_start", "Bf[None, a:b, :]", "Bf[None, 0:b - a, :]"),
    ("reverse_bwd_dy_not_reversed", "rl(C), rt(dy), D=D", "rl(C), f64(dy), D=D"),
    ("reverse_bwd_dB_not_reversed_back", 'g["dB"] = np.ascontiguousarray(g["dB"][:, ::-1])',
     'g["dB"] = np.ascontiguousarray(g["dB"])'),
    ("reverse_bwd_dx_not_reversed_back", 'g[k] = np.ascontiguousarray(g[k][:, :, ::-1])',
     'g[k] = np.ascontiguousarray(g[k])'),
    ("reverse_bwd_B_not_reversed", "rt(delta), A, rl(B), rl(C)", "rt(delta), A, f64(B), rl(C)"),
    ("varlen_bwd_reverse_ignored", "fn = self.scan_reverse_bwd if reverse else self.scan_bwd",
     "fn = self.scan_bwd"),
    ("varlen_reverse_ignored", "fn = self.scan_reverse if reverse else self.scan",
     "fn = self.scan"),
    ("conv_taps_reversed", "acc += w[None, :, k, None] * xp[:, :, k:k + L]",
     "acc += w[None, :, K - 1 - k, None] * xp[:, :, k:k + L]"),
    ("conv_halo_off_by_one", "acc += w[None, :, k, None] * xp[:, :, k:k + L]",
     "acc += w[None, :, k, None] * xp[:, :, min(k + 1, K - 1):min(k + 1, K - 1) + L]"),
    ("conv_bias_dropped", "            acc += f64(bias)[None, :, None]\n", "            pass\n"),
    ("conv_silu_is_sigmoid", "out = acc / (1.0 + np.exp(-acc)) if silu else acc\n        return out, np.ascontiguousarray(xp",
     "out = 1.0 / (1.0 + np.exp(-acc)) if silu else acc\n        return out, np.ascontiguousarray(xp"),
    ("conv_state_ignored", "st = np.zeros((b_, d_, K - 1)) if state is None else f64(state)",
     "st = np.zeros((b_, d_, K - 1))"),
    ("conv_state_out_head", "return out, np.ascontiguousarray(xp[:, :, L:])",
     "return out, np.ascontiguousarray(xp[:, :, :K - 1])"),
    ("conv_step_no_shift", "return out, np.ascontiguousarray(window[:, :, 1:])",
     "return out, np.ascontiguousarray(window[:, :, :-1])"),
]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(tmp_path, name, old, new):
    import importlib.util
    src = open(os.path.join(SRC_DIR, "__init__.py")).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / f"oracle_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    orc = mod.Oracle(oracle.build(force=False))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
