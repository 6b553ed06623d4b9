"""The pins must bite: plant one plausible mistake at a time into a copy of
the oracle's C source (CPU only), build it, and check that the pin suite
fails against it.  The committed oracle is never modified."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "arp_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("sine sign", "y[2 * p] = a * c - b * s;", "y[2 * p] = a * c + b * s;"),
    ("exclusive route", "run += (double)phi[idx];\n          theta[idx] = run;",
     "theta[idx] = run;\n          run += (double)phi[idx];"),
    ("no value un-rotation", "rotate_vec(acc, hs->theta + i * P, P, 1, out);",
     "memcpy(out, acc, sizeof(double) * (size_t)d);"),
    ("diagonal masked", "for (int64_t j = 0; j <= i; ++j) {\n    double w",
     "for (int64_t j = 0; j < i; ++j) {\n    double w"),
    ("bias sign", "scores[j] = p->scale * dot - slope * (double)(i - j);",
     "scores[j] = p->scale * dot + slope * (double)(i - j);"),
    ("scale dropped", "scores[j] = p->scale * dot - slope", "scores[j] = dot - slope"),
    ("un-rotation direction", "rotate_vec(acc, hs->theta + i * P, P, 1, out);",
     "rotate_vec(acc, hs->theta + i * P, P, 0, out);"),
    ("keys not rotated", "rotate_vec(tmp, hs->theta + j * P, P, 0, hs->krot + j * d);\n    } else {\n      memcpy(hs->krot",
     "memcpy(hs->krot + j * d, tmp, sizeof(double) * (size_t)d);\n    } else {\n      memcpy(hs->krot"),
    ("pair layout half-split", "double b = x[2 * p + 1];", "double b = x[p + npairs];"),
    ("bf16 decode shift", "<< 16;", "<< 15;"),
    ("softmax max not subtracted", "double w = exp(scores[j] - m);", "double w = exp(scores[j] - 1.0);"),
    ("gate sum includes the key's own gate", "scores[j] += gate;\n      gate += (double)lf[j];",
     "gate += (double)lf[j];\n      scores[j] += gate;"),
    ("gate sign", "scores[j] += gate;", "scores[j] -= gate;"),
]


# Mistakes in the gradients, caught by the backward pins.
BACKWARD_MUTANTS = [
    ("rotation derivative sign", "return -x[0] * a[1] + x[1] * a[0];", "return x[0] * a[1] - x[1] * a[0];"),
    ("softmax centring dropped", "const double ds = alpha[j] * (dp - Di);", "const double ds = alpha[j] * dp;"),
    ("transport angle term dropped", "g -= pair_cross(dorot + t * d + 2 * pp, otil + t * d + 2 * pp);", "(void)0;"),
    ("key gradient scale dropped", "dkt[j * d + c] += p->scale * ds * qi[c];", "dkt[j * d + c] += ds * qi[c];"),
    ("angle gradient summed forward", "for (int64_t s = L - 1; s >= 0; --s) {", "for (int64_t s = 0; s < L; ++s) {"),
    ("query gradient rotated forward", "rotate_vec(dqt + t * d, th, P, 1, oq);", "rotate_vec(dqt + t * d, th, P, 0, oq);"),
    ("upstream gradient rotated backward", "if (tv) rotate_vec(raw, hs.theta + t * P, P, 0, dorot + t * d);",
     "if (tv) rotate_vec(raw, hs.theta + t * P, P, 1, dorot + t * d);"),
    ("gate gradient one step early", "dlogf_h[j + 1] += pre;", "dlogf_h[j] += pre;"),
    ("gate gradient without the running sum", "pre += ds;", "pre = ds;"),
    ("gate left out of the recomputed logits", "alpha[j] += gate;", "(void)alpha;"),
]


# Mistakes in the on-the-fly step angles, caught by the generator pins.
GENERATOR_MUTANTS = [
    ("philox round dropped", "for (int r = 0; r < 10; ++r) {", "for (int r = 0; r < 9; ++r) {"),
    ("philox halves swapped", "c[1] = lo1;\n    c[2] = n2;\n    c[3] = lo0;",
     "c[1] = lo0;\n    c[2] = n2;\n    c[3] = lo1;"),
    ("philox key not bumped", "k1 += w1;", "(void)w1;"),
    ("counter per pair", "const uint64_t ctr[4] = {c, step, 0, 0};",
     "const uint64_t ctr[4] = {c + (uint64_t)(p % 4), step, 0, 0};"),
    ("halves of a word swapped", "(t % 2 == 0) ? (uint32_t)w : (uint32_t)(w >> 32)",
     "(t % 2 == 1) ? (uint32_t)w : (uint32_t)(w >> 32)"),
    ("uniform on [0, f_b)", "(2.0 * u - 1.0)", "u"),
]


# Mistakes in AdaScale (the per-head query scale and its schedule).
ADASCALE_MUTANTS = [
    ("head scale chain factor dropped", "for (int64_t c = 0; c < d; ++c) oq[c] *= lam;", "(void)oq;"),
    ("head scale of the next head", "return p->head_scale ? (double)p->head_scale[h] : 1.0;",
     "return p->head_scale ? (double)p->head_scale[(h + 1) % p->heads] : 1.0;"),
    ("head scale squared in the scores", "qraw[c] = lam * load_elem(", "qraw[c] = lam * lam * load_elem("),
    ("schedule takes min(L, L_ref)", "const double len = L > L_ref ? L : L_ref;",
     "const double len = L < L_ref ? L : L_ref;"),
    ("schedule in log10", "pow(log(1.0 + len / L_ref), gamma[h])", "pow(log10(1.0 + len / L_ref), gamma[h])"),
    ("schedule without the 1 +", "pow(log(1.0 + len / L_ref), gamma[h])", "pow(log(len / L_ref), gamma[h])"),
    ("schedule multiplies by tau", "gamma[h]) / tau[h];", "gamma[h]) * tau[h];"),
]


def _run_pins_against(old, new, name, tmp_path, pin_file):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutant = src.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutant)
    so_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-w",
                    "-I", os.path.join(ROOT, "oracle"), str(c_path), "-o", str(so_path), "-lm"],
                   check=True)
    env = dict(os.environ, ARP_ORACLE_LIB=str(so_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pin_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught the planted mistake {name!r}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_fail_on_planted_mistake(name, old, new, tmp_path):
    pins = "test_oracle_forget.py" if "gate" in name else "test_oracle_pins.py"
    _run_pins_against(old, new, name, tmp_path, pins)


@pytest.mark.parametrize("name,old,new", BACKWARD_MUTANTS, ids=[m[0] for m in BACKWARD_MUTANTS])
def test_backward_pins_fail_on_planted_mistake(name, old, new, tmp_path):
    _run_pins_against(old, new, name, tmp_path, "test_oracle_backward.py")


@pytest.mark.parametrize("name,old,new", GENERATOR_MUTANTS, ids=[m[0] for m in GENERATOR_MUTANTS])
def test_generator_pins_fail_on_planted_mistake(name, old, new, tmp_path):
    _run_pins_against(old, new, name, tmp_path, "test_oracle_generators.py")


@pytest.mark.parametrize("name,old,new", ADASCALE_MUTANTS, ids=[m[0] for m in ADASCALE_MUTANTS])
def test_adascale_pins_fail_on_planted_mistake(name, old, new, tmp_path):
    _run_pins_against(old, new, name, tmp_path, "test_oracle_adascale.py")
