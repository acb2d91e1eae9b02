"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
check that the pins in test_oracle_pins.py and test_oracle_backward.py catch
every one of them.

Each mutant is one textual change of moe_oracle.c; the copy is compiled to
a temporary library and the pin suite runs against it in a subprocess.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "router drops the bias": ("acc += (double)bias[i];", "acc += 0.0;"),
    "router reads noise transposed": ("acc += (double)noise[t * E + i];", "acc += (double)noise[i * T + t];"),
    "top-k ties go to the higher index": ("(best < 0 || ht[i] > ht[best])", "(best < 0 || ht[i] >= ht[best])"),
    "renorm denominator indexes the first slot":
        ("den += exp((double)ht[it[sl]] - top);", "den += exp((double)ht[it[0]] - top);"),
    "switch gate not normalised": ("gt[sl] = exp((double)ht[it[sl]] - m) / s;", "gt[sl] = exp((double)ht[it[sl]] - m);"),
    "capacity ignores k": ("cf * (double)T * (double)k / (double)E", "cf * (double)T / (double)E"),
    "capacity off by one": ("if (C < 0 || rank < C) {", "if (C < 0 || rank <= C) {"),
    "kept count not clamped": ("kept[e] = (int32_t)((C >= 0 && n > C) ? C : n);", "kept[e] = (int32_t)n;"),
    "SwiGLU gates the wrong projection": ("return (a1 / (1.0 + exp(-a1))) * a3;", "return (a3 / (1.0 + exp(-a3))) * a1;"),
    "GELU tanh approximation":
        ("return 0.5 * a1 * (1.0 + erf(a1 / sqrt(2.0)));",
         "return 0.5 * a1 * (1.0 + tanh(0.7978845608028654 * (a1 + 0.044715 * a1 * a1 * a1)));"),
    "W2 read transposed": ("acc[u] += xd[f] * (double)w2[(o0 + u) * d_ff + f];",
                           "acc[u] += xd[f] * (double)w2[f * d + o0 + u];"),
    "combine uses the slot-0 gate for every slot": ("acc += gates[t * k + s] * (double)ys", "acc += gates[t * k] * (double)ys"),
    "shared expert weighted by the slot-0 gate":
        ("moe_out += (double)ysh[(j * n + t) * d + o];", "moe_out += gates[t * k] * (double)ysh[(j * n + t) * d + o];"),
    "shared rows read token-major":
        ("moe_out += (double)ysh[(j * n + t) * d + o];", "moe_out += (double)ysh[(t * S + j) * d + o];"),
    "only the first shared expert": ("for (int64_t j = 0; j < S; ++j)", "for (int64_t j = 0; j < S && j < 1; ++j)"),
    "dropped tokens skip the shared experts":
        ("for (int64_t j = 0; j < S; ++j)", "for (int64_t j = 0; j < S && rows[t * k] >= 0; ++j)"),
    "residual left out": ("double h = res ? (double)res[t * d + o] : 0.0;", "double h = 0.0;"),
    "e4m3 ties away from zero": ("(dh == dl && ((lo + 1) & 1) == 0)", "(dh == dl)"),
    "e4m3 subnormals one binade low": ("ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    "e4m3 scale from 447": ("float si = amax / 448.0f;", "float si = amax / 447.0f;"),
    "up scale of W1 applied from W3's rows": ("a1[u] *= (double)S1[e * d_ff + f0 + u];", "a1[u] *= (double)S3[e * d_ff + f0 + u];"),
    "down scale of the block's first row for every row": ("acc[u] * (double)S2[e * d + o0 + u]", "acc[u] * (double)S2[e * d + o0]"),
    "SwiGLU derivative without the (1 + a(1 - s)) factor":
        ("a1[f] = dH * v * sg * (1.0 + u * (1.0 - sg));", "a1[f] = dH * v * sg;"),
    "GELU derivative without a * phi": ("a1[f] = dH * (Phi + u * phi);", "a1[f] = dH * Phi;"),
    "expert output gradient not gated": ("dE[q * d + o] = g[t * k + s] * (double)dy[t * d + o];",
                                         "dE[q * d + o] = (double)dy[t * d + o];"),
    "Switch gate gradient without the softmax's coupling": ("dht[i] -= pt[i] * dot;", "dht[i] -= 0.0 * dot;"),
    "aux gradient without the factor E":
        ("dht[i] += alpha_aux * pt[i] * ((double)E * fsh[i] / (double)T - dot);",
         "dht[i] += alpha_aux * pt[i] * (fsh[i] / (double)T - dot);"),
    "z gradient without the factor 2": ("alpha_z * 2.0 / (double)T", "alpha_z * 1.0 / (double)T"),
    "f counts the last slot": ("f[idx[t * k]] += 1.0;", "f[idx[t * k + k - 1]] += 1.0;"),
    "z not squared": ("zz += lse[t] * lse[t];", "zz += lse[t];"),
    "lse drops the max shift": ("lse[t] = m + log(s);", "lse[t] = log(s);"),
    "aux without the factor E": ("*aux = (double)E * a;", "*aux = a;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found exactly once"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mut), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_backward.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
