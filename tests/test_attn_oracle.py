"""CPU tests of the sparse-attention oracle: its pins (tests/attn_pins.py)
and planted mistakes in a copy of it, each of which some pin must catch."""
import os
import subprocess
import sys

import pytest

import attn_pins
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.parametrize("pin", attn_pins.PINS, ids=[p.__name__ for p in attn_pins.PINS])
def test_pin(pin):
    assert pin() == []


MUTATIONS = [
    ("scale dropped", "z[j] = P->scale * acc;", "z[j] = acc;"),
    ("sink left out of the normalizer", "if (has_sink) den += exp(s - m);", ""),
    ("window one short", "for (int64_t s = p - P->window + 1; s <= p; ++s) {",
     "for (int64_t s = p - P->window + 1; s < p; ++s) {"),
    ("window shifted", "for (int64_t s = p - P->window + 1; s <= p; ++s) {",
     "for (int64_t s = p - P->window; s < p; ++s) {"),
    ("raw position off by one", "const int64_t p = (int64_t)P->r_lens[b] - (q1 - q0) + (t - q0);",
     "const int64_t p = (int64_t)P->r_lens[b] - (q1 - q0) + (t - q0) - 1;"),
    ("query heads reversed", "const uint16_t* qrow = P->q + ((int64_t)t * H + h) * D;",
     "const uint16_t* qrow = P->q + ((int64_t)t * H + (H - 1 - h)) * D;"),
    ("value dims reversed", "acc += w[j] * bf16_value(rows[j][d]);", "acc += w[j] * bf16_value(rows[j][D - 1 - d]);"),
    ("key dims shifted", "acc += bf16_value(qrow[d]) * bf16_value(rows[j][d]);",
     "acc += bf16_value(qrow[d]) * bf16_value(rows[j][(d + 1) % D]);"),
    ("lse without the maximum", "? m + log(den) :", "? log(den) :"),
    ("out-of-contract entries kept", "if (c < 0 || c >= P->c_lens[b]) continue;", "if (c < 0) continue;"),
    ("page row ignored", "const int row = pos % page_rows;", "const int row = 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "qli_attn_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {name}"
    mutated = tmp_path / "mutated_attn.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutated.so"
    srcs = [os.path.join(ROOT, "oracle", "qli_oracle.c"), os.path.join(ROOT, "oracle", "qli_quant_oracle.c"),
            str(mutated)]
    subprocess.run(["gcc", *oracle.CFLAGS, *srcs, "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, QLI_ORACLE_LIB=str(so), PYTHONPATH=ROOT)
    code = "import sys, attn_pins; f = attn_pins.run_all(); print(f); sys.exit(1 if f else 0)"
    r = subprocess.run([sys.executable, "-W", "ignore", "-c", code], cwd=HERE, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught '{name}': {r.stdout} {r.stderr[-2000:]}"
