"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of moe_oracle.c (on the CPU, in a
temporary directory), builds it, and runs the pin tests against that build:
the run must fail.  An unmodified copy built the same way must pass."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_backward.py"),
        os.path.join(ROOT, "tests", "test_oracle_by_expert.py"),
        os.path.join(ROOT, "tests", "test_oracle_dynamic.py"),
        os.path.join(ROOT, "tests", "test_oracle_pid.py")]

MUTANTS = {
    "bias dropped": ("if (bias) s += (double)bias[e];", "if (0) s += (double)bias[e];"),
    "router weight transposed": ("s += load(x, t * d + i, dtype) * load(wr, i * E + e, dtype);",
                                 "s += load(x, t * d + i, dtype) * load(wr, e * d + i, dtype);"),
    "ties to the higher index": ("l[e] > l[best]) best = e;", "l[e] >= l[best]) best = e;"),
    "temperature multiplies": ("exp((l[e] - m) / tau)", "exp((l[e] - m) * tau)"),
    "no renormalisation": ("renorm ? p[idx[t * k + j]] / s : p[idx[t * k + j]]",
                           "p[idx[t * k + j]]"),
    "always renormalised": ("renorm ? p[idx[t * k + j]] / s : p[idx[t * k + j]]",
                            "p[idx[t * k + j]] / s"),
    "capacity floor": ("return (num + den - 1) / den;", "return num / den;"),
    "keep one too many": ("if (pos[a] >= 0 && pos[a] < C) {", "if (pos[a] >= 0 && pos[a] <= C) {"),
    "choice-major drops": (
        "for (int64_t t = 0; t < T; ++t)\n            for (int64_t j = 0; j < k; ++j) {\n"
        "                int32_t e = idx[t * k + j];",
        "for (int64_t j = 0; j < k; ++j)\n            for (int64_t t = 0; t < T; ++t) {\n"
        "                int32_t e = idx[t * k + j];"),
    "choice order ignored": (
        "for (int64_t j = 0; j < k; ++j)\n            for (int64_t t = 0; t < T; ++t) {\n"
        "                int32_t e = idx[t * k + j];",
        "for (int64_t t = 0; t < T; ++t)\n            for (int64_t j = 0; j < k; ++j) {\n"
        "                int32_t e = idx[t * k + j];"),
    "load deviation signed": ("double ad = diff < 0 ? -diff : diff;", "double ad = diff;"),
    "load CV with E - 1": ("sqrt(ss / (double)E)", "sqrt(ss / (double)(E - 1))"),
    "mean load over busy experts": ("double m = sum / (double)E;",
                                    "double m = sum / (double)(E - empty);"),
    "MLP router W1 transposed": ("s += v[j] * load(w1, j * m + n, dtype);",
                                 "s += v[j] * load(w1, n * r + j, dtype);"),
    "RMS norm over the sum": ("double inv = 1.0 / sqrt(ss / (double)r + eps);",
                              "double inv = 1.0 / sqrt(ss + eps);"),
    "depth average subtracted": ("if (prev) s += gamma * load(prev, t * r + j, dtype);",
                                 "if (prev) s -= gamma * load(prev, t * r + j, dtype);"),
    "no GELU on the second layer": ("b[n] = gelu(s);", "b[n] = s;"),
    "router output bias dropped": ("if (b3) s += (double)b3[e];", "if (0) s += (double)b3[e];"),
    "GELU derivative without the density term": (
        "+ v * exp(-0.5 * v * v) / sqrt(2.0 * M_PI);", "+ 0.0 * v;"),
    "renormalised gate gradient without the shared term": (
        "dp[idx[t * k + j]] = (dga[t * k + j] - sg) / S;", "dp[idx[t * k + j]] = dga[t * k + j] / S;"),
    "softmax backward without the temperature": (
        "dl[t * E + e] = p[e] * (dp[e] - pd) / tau;", "dl[t * E + e] = p[e] * (dp[e] - pd);"),
    "expert output gradient without the gate": (
        "dO[c] = gate[a] * dy[t * d + c];", "dO[c] = dy[t * d + c];"),
    "router path missing from dx": (
        "for (int64_t e = 0; e < E; ++e) s += dl[t * E + e] * load(wr, i * E + e, dtype);", ""),
    "tanh GELU": ("0.5 * v * (1.0 + erf(v / sqrt(2.0)))",
                  "0.5 * v * (1.0 + tanh(0.7978845608028654 * (v + 0.044715 * v * v * v)))"),
    "GELU on the up branch": ("g[n] = gelu(g[n]) * u[n];", "g[n] = g[n] * gelu(u[n]);"),
    "down weight transposed": ("o[c] += g[n] * load(wd, wrow + c, dtype);",
                               "o[c] += g[n] * load(wd, (e * d + c) * d_ff + n, dtype);"),
    "expert index ignored": ("int64_t t = tok[r], e = ex[r];", "int64_t t = tok[r], e = 0;"),
    "second expert dropped in combine": ("for (int64_t j = 0; j < k; ++j)\n                if (row_of",
                                         "for (int64_t j = 0; j < 1; ++j)\n                if (row_of"),
    "padded layout one expert short": (
        "offset[e + 1] = layout == 1 ? (int32_t)((e + 1) * C)",
        "offset[e + 1] = layout == 1 ? (int32_t)(e * C)"),
    "single-entry down gradient without the gate": (
        "acc += gate[s] * (act * u) * dy[t * d + b];", "acc += (act * u) * dy[t * d + b];"),
    "single-entry gate gradient with GELU for its derivative": (
        "xa * dh * u * gelu_grad(g)", "xa * dh * u * gelu(g)"),
    "router backward without the temperature": (
        "dl[t * E + e] = q[e] * (dq[e] - qd) / tau;", "dl[t * E + e] = q[e] * (dq[e] - qd);"),
    "router backward renormalisation without the shared term": (
        "dq[it[j]] = (dgate[t * k + j] - dot) / S;", "dq[it[j]] = dgate[t * k + j] / S;"),
    "router backward softmax unnormalised": ("q[e] = q[e] / zs;", "q[e] = q[e];"),
    "dynamic count: strict threshold": ("if (j + 1 >= kmin && mass >= theta)",
                                        "if (j + 1 >= kmin && mass > theta)"),
    "dynamic count: floor ignored": ("if (j + 1 >= kmin && mass >= theta)", "if (mass >= theta)"),
    "dynamic count: gates renormalised over every slot": (
        "for (int64_t j = 0; j < kt; ++j) s += p[it[j]];",
        "for (int64_t j = 0; j < kmax; ++j) s += p[it[j]];"),
    "dynamic count: unused slots keep their expert": ("it[j] = -1;", "(void)0;"),
    "dynamic backward: unused slots counted as expert 0": (
        "if (idx[t * k + j] >= 0) S += p[idx[t * k + j]];",
        "S += p[idx[t * k + j] < 0 ? 0 : idx[t * k + j]];"),
    "dynamic router backward: unused slots counted as expert 0": (
        "if (it[j] >= 0) S += q[it[j]];", "S += q[it[j] < 0 ? 0 : it[j]];"),
    "PID error sign flipped": (
        "double err = mean > 0 ? (mean - (double)count[e]) / mean : 0.0;",
        "double err = mean > 0 ? ((double)count[e] - mean) / mean : 0.0;"),
    "PID error not relative": (
        "double err = mean > 0 ? (mean - (double)count[e]) / mean : 0.0;",
        "double err = mean > 0 ? (mean - (double)count[e]) : 0.0;"),
    "PID integral not accumulated": ("double integral = state[e] + err;", "double integral = err;"),
    "PID derivative reversed": ("double deriv = err - state[E + e];",
                                "double deriv = state[E + e] - err;"),
    "PID warmup scale skips the derivative": (
        "bias[e] = scale * ((p_term + i_term) + d_term);",
        "bias[e] = scale * (p_term + i_term) + d_term;"),
    "PID previous error not kept": ("state[E + e] = err;", "state[E + e] = 0.0;"),
    "realised capacity floor": ("return num / den + (num % den != 0);", "return num / den;"),
    "realised capacity from the token count": ("int64_t num = cap_num * A, den = cap_den * E;",
                                               "int64_t num = cap_num * T, den = cap_den * E;"),
}


def _run(name, src_text, tmp):
    path = os.path.join(tmp, name.replace(" ", "_"))
    os.makedirs(path, exist_ok=True)
    c = os.path.join(path, "m.c")
    lib = os.path.join(path, "libm.so")
    open(c, "w").write(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-std=c11", c, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_is_caught():
    base = open(SRC).read()
    for name, (old, new) in MUTANTS.items():
        assert base.count(old) == 1, f"mutation site for {name!r} not unique in the source"
    with tempfile.TemporaryDirectory() as tmp:
        jobs = {"(unmodified)": base}
        jobs.update({n: base.replace(o, w) for n, (o, w) in MUTANTS.items()})
        with ThreadPoolExecutor(max_workers=4) as ex:
            rc = dict(zip(jobs, ex.map(lambda kv: _run(kv[0], kv[1], tmp), jobs.items())))
    assert rc.pop("(unmodified)") == 0
    survivors = [n for n, code in rc.items() if code == 0]
    assert not survivors, f"pins missed planted mistakes: {survivors}"
