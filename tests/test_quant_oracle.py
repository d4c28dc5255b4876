"""Pins of the query-quantization and index-K write oracle (CPU).

The pages give no formula for the quantization (Guide, 数据流: each Q head
becomes INT8 with a representable FP16 scale; per-token K scale), so the
oracle's reading is pinned by closed forms and by properties any symmetric
INT8 quantizer with that scale must have, chosen so that a wrong divisor,
a dropped rounding of the scale, a wrong rounding rule, a missing clamp or
a wrong scatter address fails one of them."""
import numpy as np
import pytest

import oracle


def f32_to_bf16_bits(x):
    """Bit patterns of float32 values that are exact in bfloat16."""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bfloat16"
    return (u >> 16).astype(np.uint16)


def test_amax_127_means_unit_scale_and_plain_rounding():
    # amax = 127 -> s = 1.0 exactly, q = round-half-even(x)
    x = np.zeros((1, 128), np.float32)
    vals = [127, -64, 0.5, 1.5, 2.5, -0.5, -1.5, -126.5, 100.25, 3.75]
    x[0, :len(vals)] = vals
    q, s = oracle.quantize_rows(x)
    assert s[0] == 0x3C00
    assert list(q[0, :len(vals)]) == [127, -64, 0, 2, 2, 0, -2, -126, 100, 4]
    assert np.all(q[0, len(vals):] == 0)


def test_power_of_two_scales_are_exact():
    # amax = 127 * 2^k -> s = 2^k exactly and q = rint(x / 2^k)
    rng = np.random.default_rng(1)
    for k in (-10, -3, 0, 4, 9):
        base = rng.integers(-127, 128, size=128).astype(np.float32)
        base[5] = 127.0
        x = (base * np.float32(2.0 ** k))[None, :]
        q, s = oracle.quantize_rows(x)
        assert oracle.f16_value(s)[0] == 2.0 ** k
        assert np.array_equal(q[0], base.astype(np.int8))


def test_zero_row_and_sign_symmetry():
    q, s = oracle.quantize_rows(np.zeros((3, 128), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    rng = np.random.default_rng(2)
    x = rng.normal(0, 3, size=(50, 128)).astype(np.float32)
    q1, s1 = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows(-x)
    assert np.array_equal(s1, s2) and np.array_equal(q1, -q2)


def test_doubling_the_row_doubles_the_scale_only():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, size=(40, 128)).astype(np.float32)
    q1, s1 = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows(x * 2)
    assert np.array_equal(q1, q2)
    assert np.array_equal(oracle.f16_value(s2), 2 * oracle.f16_value(s1))


def test_scale_error_and_reconstruction_bounds():
    rng = np.random.default_rng(4)
    x = (rng.normal(0, 1, size=(300, 128)) * rng.uniform(0.01, 50, size=(300, 1))).astype(np.float32)
    q, s = oracle.quantize_rows(x)
    sv = oracle.f16_value(s)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    # the scale is amax/127 up to one FP32 and one FP16 rounding
    assert np.all(np.abs(sv - amax / 127) <= (2.0 ** -11 + 2.0 ** -23) * amax / 127)
    # the largest element maps to +-127; every element reconstructs within
    # half a step (plus the scale's own relative error), and |q| <= 127
    i = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(300), i]) == 127)
    err = np.abs(q * sv[:, None] - x)
    bound = 0.5 * sv[:, None] * (1 + 2.0 ** -10) + 127 * sv[:, None] * 2.0 ** -10
    assert np.all(err <= bound)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)


def clamp_rows():
    """Rows whose scale leaves the FP16 normal range: tiny rows (the scale is
    an FP16 subnormal, rounded by up to half of 2^-24) and huge rows (the
    scale saturates at 65504), where amax / s exceeds 127.5."""
    rows = []
    for t in (1.2, 1.4, 1.45, 2.3, 2.45, 3.4):
        rows.append(np.float32(127 * t * 2.0 ** -24))
    rows += [np.float32(127 * 70000.0), np.float32(127 * 65504.0 * 1.01)]
    x = np.zeros((len(rows), 128), np.float32)
    x[:, 0] = rows
    x[:, 1] = -np.array(rows, np.float32)
    return x


def test_clamp_outside_the_fp16_normal_range():
    x = clamp_rows()
    q, s = oracle.quantize_rows(x)
    sv = oracle.f16_value(s)
    ratio = x[:, 0] / sv
    assert np.any(ratio > 127.5)              # the clamp is exercised
    assert np.all(q[:, 0] == 127) and np.all(q[:, 1] == -127)
    assert np.all(s[-2:] == 0x7BFF)           # saturated scale, not inf


def test_scale_is_rounded_before_dividing():
    # amax = 127 (1 - 2^-13): fp32(amax/127) = 1 - 2^-13 rounds to the FP16
    # scale 1.0, so 2.5 is an exact tie (-> 2); dividing by the unrounded
    # scale would give 2.5003 (-> 3)
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = np.float32(127 * (1 - 2.0 ** -13))
    x[0, 1] = 2.5
    x[0, 2] = -3.5
    q, s = oracle.quantize_rows(x)
    assert s[0] == 0x3C00
    assert list(q[0, :3]) == [127, 2, -4]


def test_bf16_input_equals_float32_of_the_same_values():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 2, size=(64, 128)).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # exact in bf16
    q1, s1 = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows(f32_to_bf16_bits(x))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_weight_rounding_is_ieee_rne():
    rng = np.random.default_rng(6)
    w = np.concatenate([rng.normal(0, 0.1, 5000), rng.normal(0, 1e4, 200),
                        [65504.0, 65519.0, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26]])
    w = w.astype(np.float32)
    got = oracle.round_weights(w)
    with np.errstate(over="ignore"):
        want = w.astype(np.float16).view(np.uint16)  # numpy: IEEE RNE, overflow to inf
    assert np.array_equal(got, want)


def test_write_k_scatter_by_brute_force():
    rng = np.random.default_rng(7)
    P, R = 5, 64
    kp = np.full((P, R, 128), 127, np.int8)
    sp = np.full((P, R), 60000, np.uint16)
    x = rng.normal(0, 1, size=(9, 128)).astype(np.float32)
    slot = np.array([0, 63, 64, 3 * R + 7, -1, P * R, P * R - 1, 130, -5], np.int64)
    k2, s2 = oracle.write_k(x, slot, kp, sp)
    q, sc = oracle.quantize_rows(x)
    touched = set()
    for i, sl in enumerate(slot):
        if 0 <= sl < P * R:
            pg, row = divmod(int(sl), R)
            assert np.array_equal(k2[pg, row], q[i]) and s2[pg, row] == sc[i]
            touched.add((pg, row))
    for pg in range(P):
        for row in range(R):
            if (pg, row) not in touched:
                assert np.all(k2[pg, row] == 127) and s2[pg, row] == 60000


QUANT_MUTATIONS = [
    ("divisor 128", "float s32 = amax / 127.0f;", "float s32 = amax / 128.0f;"),
    ("scale not rounded before dividing",
     "float s = (float)oracle_f16_value(sh);", "float s = s32;"),
    ("ties away from zero", "float r = rintf(", "float r = roundf("),
    ("no clamp", "if (r > 127.0f) r = 127.0f;", ""),
    ("scale overflows to inf", "if ((sh & 0x7FFFu) == 0x7C00u) sh = 0x7BFFu; /* saturate */", ""),
    ("scatter row stride", "memcpy(kpages + s * QDIM, q, QDIM);",
     "memcpy(kpages + (s ^ 1) * QDIM, q, QDIM);"),
    ("weights truncated", "out[i] = oracle_f16_round((double)load_value(w, dtype, i));",
     "out[i] = oracle_f16_round((double)(float)(int)(load_value(w, dtype, i) * 1024.0f) / 1024.0);"),
]


@pytest.mark.parametrize("name,old,new", QUANT_MUTATIONS, ids=[m[0] for m in QUANT_MUTATIONS])
def test_quant_mutation_is_caught(name, old, new, tmp_path):
    """Plant a plausible mistake in a copy of the quantization oracle; some
    pin of this file must fail on it."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    src = open(os.path.join(root, "oracle", "qli_quant_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {name}"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutated.so"
    subprocess.run(["gcc", *oracle.CFLAGS, os.path.join(root, "oracle", "qli_oracle.c"), str(mutated),
                    "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, QLI_ORACLE_LIB=str(so), PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(here, "test_quant_oracle.py"), "-k", "not mutation"],
                       cwd=root, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught '{name}': {r.stdout[-1500:]}"
