"""The score kernels never form qk/1024 directly: the INT8 MFMA accumulates
q.k on top of the bits of 4.0f, and the epilogue reads the sum back as a
float.  These CPU tests check, bit for bit and for every q.k that int8
operands can produce, that the two epilogue forms the kernels use give the
golden FP16 steps (fp16(qk/1024), ReLU, fp16(x * m)):

- plain form: fp16(2048 * F - 8192), then the ReLU on the fp16 value;
- scaled form: y = clamp(F - 4, 0, 1) (the ReLU folded into the clamp),
  fp16(y), then the product with the multiplier held as m * 2^11, valid for
  every fp16 m with |m| < 32.

The golden side is the definition: one round-to-nearest-even of the exact
quotient to fp16, max with +0, and one fp16 rounding of the exact product
(numpy's float16 multiply rounds the exact float32 product of two fp16
values once)."""
import numpy as np
import pytest

SEED_BITS = 0x40800000  # 4.0f
QK_MIN = -128 * 127 * 128   # -2080768: q = -128 against k = 127 on all 128 dims
QK_MAX = 128 * 128 * 128    # +2^21: q = k = -128 on all 128 dims


def _all_qk():
    return np.arange(QK_MIN, QK_MAX + 1, dtype=np.int64)


def _accumulator_float(qk):
    """The float whose bits are the seed plus q.k (int32 wrap-free here)."""
    return (np.int64(SEED_BITS) + qk).astype(np.uint32).view(np.float32)


def _golden_x(qk):
    """max(fp16(qk / 1024), +0) from the exact quotient (one rounding)."""
    x = (qk.astype(np.float64) / 1024.0).astype(np.float16)
    return np.where(x > 0, x, np.float16(0.0))


def test_accumulator_reads_back_qk():
    qk = _all_qk()
    F = _accumulator_float(qk)
    pos = qk >= 0
    # q.k >= 0: F is exactly 4 + qk * 2^-21
    assert np.array_equal(F[pos].astype(np.float64), 4.0 + qk[pos].astype(np.float64) * 2.0 ** -21)
    # q.k < 0: F lies in [2, 4), below the seed
    assert np.all((F[~pos] >= 2.0) & (F[~pos] < 4.0))


def test_plain_form_equals_golden_relu():
    qk = _all_qk()
    F = _accumulator_float(qk)
    # one fma: 2048 * F - 8192 is exact in FP32 for these F, then one RNE to fp16
    v = (np.float64(2048.0) * F.astype(np.float64) - 8192.0).astype(np.float32)
    x = v.astype(np.float16)
    x = np.where(x.view(np.int16) > 0, x, np.float16(0.0))  # ReLU on the fp16 bits
    assert np.array_equal(x.view(np.uint16), _golden_x(qk).view(np.uint16))


def _scaled_y(qk):
    F = _accumulator_float(qk)
    y = F - np.float32(4.0)  # exact (Sterbenz / same binade)
    return np.clip(y, np.float32(0.0), np.float32(1.0)).astype(np.float16)


def test_scaled_form_is_golden_x_times_2_pow_minus_11():
    qk = _all_qk()
    y = _scaled_y(qk)
    gx = _golden_x(qk)
    # fp16(y) is the golden x scaled by 2^-11, exactly (subnormal y included)
    assert np.array_equal(y.astype(np.float64) * 2048.0, gx.astype(np.float64))


def _multipliers():
    """fp16 multipliers across the range the scaled form accepts: every
    binade from the smallest subnormal to just below 32, both signs, the
    largest fp16 below 32, zero and -0."""
    rng = np.random.default_rng(7)
    bits = np.concatenate([
        np.arange(1, 0x0400, 37, dtype=np.uint16),                    # subnormals
        rng.integers(0x0400, 0x5000, size=160, dtype=np.uint16),      # normals below 32
        np.array([0x4FFF, 0x4FFE, 0x3C00, 0x0001, 0x03FF, 0x0400, 0x0000], np.uint16),
    ])
    bits = np.concatenate([bits, bits | np.uint16(0x8000)])
    return bits.view(np.float16)


@pytest.mark.parametrize("chunk", range(4))
def test_scaled_products_equal_golden_products(chunk):
    qk = _all_qk()
    y = _scaled_y(qk)
    gx = _golden_x(qk)
    ms = _multipliers()
    ms = ms[chunk::4]
    for m in ms:
        ms11 = (np.float64(m) * 2048.0)
        assert np.float16(ms11).astype(np.float64) == ms11  # m * 2^11 is an exact fp16
        got = y * np.float16(ms11)
        want = gx * m
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), float(m)


def test_multiplier_bound_is_tight():
    """m = 32 is the first multiplier whose 2^11 multiple overflows fp16, so
    the kernels take the plain form for it (and for larger |m|)."""
    with np.errstate(over="ignore"):
        assert np.isfinite(np.float16(31.984375 * 2048.0))
        assert np.isinf(np.float16(32.0 * 2048.0))
