"""The seeded input recipes: determinism, shapes and bf16 rounding (CPU only)."""
import numpy as np

import ssm_workloads as W


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5, 0.0, 3.0e38], np.float32)
    bits = W.bf16_bits(vals)
    # 1+2^-8 is a tie between 1.0 and 1+2^-7: even mantissa wins (1.0)
    assert [hex(b) for b in bits[:3]] == ["0x3f80", "0x3f80", "0x3f82"]
    assert bits[3] == 0x3F80
    back = W.bf16_to_f32(bits)
    assert back[4] == -2.5 and back[5] == 0.0
    # every bf16 value widens exactly and re-rounds to itself
    allbits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(W.bf16_bits(W.bf16_to_f32(allbits)), allbits)


def test_recipes_deterministic_and_shaped():
    a = W.scan_prefill(batch=1, seqlen=33, dim=40)
    b = W.scan_prefill(batch=1, seqlen=33, dim=40)
    for k in a.arrays:
        assert np.array_equal(a.arrays[k], b.arrays[k]), k
    assert a.arrays["x"].shape == (1, 33, 40) and a.arrays["x"].dtype == np.uint16
    assert a.arrays["conv_w"].shape == (40, 4)
    assert np.array_equal(a.arrays["A"][3], -np.arange(1, 17, dtype=np.float32))
    t = W.scan_tiny()
    assert t.arrays["x"].shape == (1, 64, 16) and t.arrays["x"].dtype == np.float32
    s = W.ssd_long(seqlen=256, nheads=3, headdim=8, d_state=16)
    assert s.arrays["x"].shape == (1, 256, 3, 8) and np.all(s.arrays["A"] < 0)
    assert np.all(s.arrays["A"] >= -16.0 - 1e-5) and np.all(s.arrays["A"] <= -1.0 + 1e-6)
    d = W.decode_stream(batch=2, dim=8, prefill=3, steps=2)
    assert d.arrays["x"].shape == (5, 2, 8)


def test_saturation_of_default_recipe():
    """With the stated generators nearly every dt pre-activation lies above
    softplus^-1(0.1) = -2.2522, so dt sits on the upper clip; the unsaturated
    variant spreads it over both clip edges."""
    p = W.scan_tiny(seqlen=4096, dim=64)
    pre = p.arrays["dt_w"][None, None, :] * p.arrays["dt"][..., None] + p.arrays["dt_bias"]
    assert np.mean(pre >= -2.2522) > 0.98
    q = W.scan_tiny(seqlen=4096, dim=64, unsaturated=True)
    pre = q.arrays["dt_w"][None, None, :] * q.arrays["dt"][..., None] + q.arrays["dt_bias"]
    assert 0.05 < np.mean(pre >= -2.2522) < 0.5 and np.mean(pre <= -6.9073) > 0.01


def test_a_init_forms():
    """The three forms of A: the exact diagonal, the same initialisation as a
    model stores it (fp32 log then fp32 exp: the entries for 5, 10, 11, 13 and
    15 land an ulp or two off, so A is no longer a run of multiples of its first
    entry), and independent random rows; the other draws are unchanged."""
    base = W.scan_bulk(batch=1, seqlen=8, dim=64)
    li = W.scan_bulk(batch=1, seqlen=8, dim=64, a_init="log_init")
    rnd = W.scan_bulk(batch=1, seqlen=8, dim=64, a_init="random")
    diag = -np.arange(1, 17, dtype=np.float32)
    assert np.array_equal(base.arrays["A"][5], diag)
    off = np.nonzero(li.arrays["A"][0] != diag)[0] + 1
    assert list(off) == [5, 10, 11, 13, 15]
    assert np.all(np.abs(li.arrays["A"][0] - diag) <= 2 * np.spacing(np.abs(diag)))
    assert np.array_equal(li.arrays["A"][0], li.arrays["A"][63])
    A = rnd.arrays["A"]
    assert A.shape == (64, 16) and np.all(A <= -1.0) and np.all(A >= -16.0)
    assert len(np.unique(A)) == A.size
    for k in base.arrays:
        if k != "A":
            assert np.array_equal(base.arrays[k], li.arrays[k]) and np.array_equal(base.arrays[k], rnd.arrays[k]), k
