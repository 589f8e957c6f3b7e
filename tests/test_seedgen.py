"""The seeded input generator against its published definition (CPU only)."""
import math
import struct

import numpy as np

import seedgen

MASK = (1 << 64) - 1


def py_sm64(x):
    """Vigna's splitmix64 step, written out independently in Python integers."""
    z = (x + 0x9E3779B97F4A7C15) & MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def py_bf16_rne(f64):
    """fp64 -> fp32 (struct packs with round-to-nearest-even) -> bf16 by exact tie-to-even rule."""
    (u,) = struct.unpack("<I", struct.pack("<f", f64))
    upper, lower = u >> 16, u & 0xFFFF
    if lower > 0x8000 or (lower == 0x8000 and (upper & 1)):
        upper += 1
    return upper & 0xFFFF


def test_splitmix64_published_sequence():
    # splitmix64 seeded with 0 starts 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F
    # (the generator's state advances by the golden gamma; sm64(x) is the output for state x).
    gamma = 0x9E3779B97F4A7C15
    assert seedgen.sm64(0) == 0xE220A8397B1DCDAF
    assert seedgen.sm64(gamma) == 0x6E789E6AA1B965F4
    assert seedgen.sm64((2 * gamma) & MASK) == 0x06C45D188009454F
    for x in (1, 12345, MASK, 0x5EED0003):
        assert seedgen.sm64(x) == py_sm64(x)


def test_elements_match_independent_definition():
    seed = 0x5EED0002
    for t in ("q", "k", "v", "do"):
        key = py_sm64(seed ^ (seedgen.TENSOR_IDS[t] << 56))
        assert seedgen.stream_key(seed, t) == key
        got = seedgen.normal_bf16(seed, t, (3, 5, 7))
        flat = got.reshape(-1)
        for n in (0, 1, 2, 50, 104):
            x = py_sm64((key + n) & MASK)
            u1 = ((x >> 32) + 1) / 2.0 ** 32
            u2 = (x & 0xFFFFFFFF) / 2.0 ** 32
            z = math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2)
            assert flat[n] == py_bf16_rne(z), (t, n)
        # an offset window reproduces the same elements
        win = seedgen.normal_bf16(seed, t, (10,), start=40)
        assert np.array_equal(win, flat[40:50])


def test_bf16_round_to_nearest_even():
    cases = {1.0: 0x3F80, 1.00390625: 0x3F80, 1.01171875: 0x3F82, -2.0: 0xC000,
             1.0078125: 0x3F81, 3.140625: 0x4049, 1e-40: 0x0001}
    for f, bits in cases.items():
        assert seedgen.f32_to_bf16_bits(f) == bits, (f, hex(seedgen.f32_to_bf16_bits(f)))


def test_distribution_is_standard_normal():
    from scipy import stats
    x = seedgen.bf16_bits_to_f64(seedgen.normal_bf16(0x5EED0001, "q", (1 << 20,)))
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert stats.kstest(x[:200000], "norm").pvalue > 1e-3


def test_threads_do_not_change_bytes():
    a = seedgen.normal_bf16(7, "v", (300000,), threads=1)
    b = seedgen.normal_bf16(7, "v", (300000,), threads=8)
    assert np.array_equal(a, b)


def test_row_sample():
    N = 8192
    r = seedgen.sample_rows(0x5EED0003, 5, N, 256)
    assert r.shape == (256,)
    assert np.all(np.diff(r) > 0)
    assert set(range(16)) <= set(r.tolist()) and (N - 1) in r
    assert np.array_equal(r, seedgen.sample_rows(0x5EED0003, 5, N, 256))
    assert not np.array_equal(r, seedgen.sample_rows(0x5EED0003, 6, N, 256))
    assert np.array_equal(seedgen.sample_rows(1, 0, 100, 256), np.arange(100))
    allr = seedgen.sample_rows_all(1, 4, 300, 20)
    assert allr.shape == (4, 20)


# ---------------------------------------------------------------- FP8 E4M3FN encoding

def test_e4m3_decoder_anchor_values():
    """Values fixed by the E4M3FN definition (bias 7, 3 mantissa bits, no infinities)."""
    dec = seedgen.e4m3_to_f64
    assert dec(np.array([0x38]))[0] == 1.0 and dec(np.array([0xB8]))[0] == -1.0
    assert dec(np.array([0x7E]))[0] == 448.0 and dec(np.array([0x01]))[0] == 2.0 ** -9
    assert dec(np.array([0x08]))[0] == 2.0 ** -6 and dec(np.array([0x07]))[0] == 7 * 2.0 ** -9
    assert dec(np.array([0x3C]))[0] == 1.5 and dec(np.array([0x40]))[0] == 2.0
    assert np.isnan(dec(np.array([0x7F]))[0]) and np.isnan(dec(np.array([0xFF]))[0])
    finite = dec(np.arange(256, dtype=np.uint8))
    pos = np.sort(finite[(finite > 0) & np.isfinite(finite)])
    assert len(pos) == 126 and np.all(np.diff(pos) > 0)   # 126 distinct positive values


def test_e4m3_encoder_round_trip_and_rne():
    enc, vals = seedgen.f64_to_e4m3, seedgen.E4M3_VALUES
    for code in range(256):
        if code in (0x7F, 0xFF):
            continue
        assert enc(vals[code]) == code, hex(code)
    pos = [(vals[c], c) for c in range(1, 0x7F)]
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        want = ca if ca % 2 == 0 else cb         # ties to the even code (even mantissa)
        assert enc(mid) == want, (a, b)
        assert enc(-mid) == want | 0x80
        assert enc(mid * (1 - 1e-12)) == ca and enc(mid * (1 + 1e-12)) == cb
    assert enc(1000.0) == 0x7E and enc(-1e30) == 0xFE and enc(449.0) == 0x7E   # saturation
    assert enc(2.0 ** -10) == 0x00 and enc(2.0 ** -10 * 1.001) == 0x01          # below the smallest subnormal


def test_e4m3_stream_matches_normals():
    """The FP8 stream quantises the same N(0,1) values as the bf16 stream."""
    codes = seedgen.normal_e4m3(11, "k", (4096,), 32.0)
    bf = seedgen.bf16_bits_to_f64(seedgen.normal_bf16(11, "k", (4096,)))
    vals = seedgen.e4m3_to_f64(codes) / 32.0
    assert np.all(np.isfinite(vals))
    # both are within their format's half-ulp of the same normal value
    assert np.max(np.abs(vals - bf) / np.maximum(np.abs(bf), 2.0 ** -6 / 32)) < 2 ** -4 + 2 ** -8
