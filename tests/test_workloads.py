"""The seeded input generators (CPU): deterministic, the stated shapes and
encodings, and slots that address each request's own pages."""
import numpy as np

import qli_workloads as W


def test_bf16_encoding_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.4e38], np.float32)
    b = W.bf16_bits(x)
    # exact, tie to even (down), tie to even (up), exact, below half, overflow to inf
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80, 0x7F80]
    assert np.array_equal(W.bf16_to_f32(b[:4]), np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], np.float32))


def test_activations_are_seeded_and_shaped():
    a = W.make_activations(3, 1, 50, "bf16")
    b = W.make_activations(3, 1, 50, "bf16")
    c = W.make_activations(4, 1, 50, "bf16")
    assert a.dtype == np.uint16 and a.shape == (50, 128)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    f = W.make_activations(3, 1, 50, "f32")
    assert f.dtype == np.float32 and np.all(np.isfinite(f))
    assert np.array_equal(W.bf16_bits(f), a)          # the bf16 rows are the f32 rows rounded
    k = W.make_activations(3, 1, 50, "f32", which="k")
    assert not np.array_equal(k, f)                   # K and Q streams differ
    w = W.make_head_weights(3, 1, 1000, "f32")
    assert abs(float(w.std()) - 0.1) < 0.01


def test_request_slots_follow_the_block_table():
    pb = W.tiny()
    R = pb.page_rows
    slots = W.request_slots(pb.block_table, pb.k_lens, pb.ratio)
    assert len(slots) == int(pb.k_lens.sum())
    for j, sl in enumerate(slots):                    # tiny has one request
        assert sl == int(pb.block_table[0, j // R]) * R + j % R
    # the slots hold the request's K rows in the generated pool
    rows = pb.k_pages.reshape(-1, 128)[slots]
    assert not np.any(np.all(rows == 127, axis=1))    # no poisoned row is addressed
