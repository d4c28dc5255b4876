"""Plant plausible mistakes in a copy of the oracle, on the CPU, and check
that the pins catch every one of them (a pin that passes on a broken oracle
pins nothing)."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTATIONS = [
    ("scale 1000 instead of 1024", "(double)acc / 1024.0", "(double)acc / 1000.0"),
    ("ReLU dropped", "if (!(oracle_f16_value(x) > 0.0)) x = 0;", ""),
    ("last head dropped", "for (int h = 0; h < N; ++h) {\n    const int8_t* qrow",
     "for (int h = 0; h < N - 1; ++h) {\n    const int8_t* qrow"),
    ("K dim index", "(int32_t)krow[d]", "(int32_t)krow[d ^ 1]"),
    ("heads reversed against their multipliers", "((int64_t)t * N + h) * ORACLE_HEAD_DIM",
     "((int64_t)t * N + (N - 1 - h)) * ORACLE_HEAD_DIM"),
    ("tie-break reversed", "return (a->id > b->id) - (a->id < b->id);",
     "return (a->id < b->id) - (a->id > b->id);"),
    ("last block not pinned", "chosen[others] = last;", "chosen[others] = 0;"),
    ("causal off by one", "int64_t V = (p + 1) / P->ratio;", "int64_t V = p / P->ratio;"),
    ("K scale dropped", "float score = sum * kscale;", "float score = sum;"),
    ("q_scale dropped", "oracle_f16_value(P->weights[o]) * oracle_f16_value(P->q_scale[o])",
     "oracle_f16_value(P->weights[o])"),
    ("head sum in fp16", "sum = sum + (float)pv;",
     "sum = (float)oracle_f16_value(oracle_f16_round((double)sum + pv));"),
    ("block min instead of max", "if (score[j] > m) m = score[j];",
     "if (score[j] < m) m = score[j];"),
    ("candidate block missing its last position",
     "j < (c + 1) * ORACLE_BLOCK && j < V; ++j) eligible[j] = 1;",
     "j < (c + 1) * ORACLE_BLOCK - 1 && j < V; ++j) eligible[j] = 1;"),
    ("product not rounded to fp16",
     "uint16_t p = oracle_f16_round(oracle_f16_value(x) * oracle_f16_value(mh[h])); /* FP16 */\n"
     "    double pv = oracle_f16_value(p);",
     "uint16_t p = oracle_f16_round(oracle_f16_value(x) * oracle_f16_value(mh[h])); /* FP16 */\n"
     "    double pv = oracle_f16_value(x) * oracle_f16_value(mh[h]);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "qli_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {name}"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutated.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, QLI_ORACLE_LIB=str(so), PYTHONPATH=ROOT)
    code = "import sys, pins; f = pins.run_all(); print(f); sys.exit(1 if f else 0)"
    r = subprocess.run([sys.executable, "-W", "ignore", "-c", code], cwd=HERE, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"no pin caught '{name}': {r.stdout} {r.stderr[-2000:]}"
