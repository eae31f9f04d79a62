"""Pins of the oracle's grouped 8- and 4-bit KV quantisation.

Byte budgets, footprints and the read/convert trade-off are checked against
the numbers the inference-optimization chapter prints (tests/golden/
kv_quant.txt).  The code arithmetic, which the pages leave open, is checked
against exact rational arithmetic: every code is a nearest integer of
x / scale, the scale is the half nearest max|x| / qmax, round trips of
values on the code grid are exact, and the error of a round trip is at most
half a scale step.  Planted mistakes must each fail a pin.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import quant as qt


def _f(x):
    return [float(v) for v in x]


def test_group_bytes_and_footprints(golden):
    g = golden("kv_quant.txt")
    for fmt, nbytes, bits in g["group"]:
        assert qt.group_bytes(fmt) == int(nbytes)
        assert qt.bits_per_value(fmt) == Fraction(bits)
    for fmt, bf16, quant, saved in g["context"]:
        q = qt.quantized_bytes(int(bf16), fmt)
        assert q == int(quant) and int(bf16) - q == int(saved)
    for fmt, bf16, quant, n, total_gib in g["request"]:
        q = qt.quantized_bytes(int(bf16), fmt)
        assert q == Fraction(quant)
        assert abs(float(q) * int(n) / 1024 - float(total_gib)) < 0.005


def test_read_saving_and_crossover(golden):
    g = golden("kv_quant.txt")
    for saved_mib, tbps, read_ms, tc, net in g["saving"]:
        # the page rounds the read time ("about"); 540 MiB / 1.16 TB/s = 0.4881 ms
        read = float(saved_mib) * 2**20 / (float(tbps) * 1e12) * 1e3
        assert abs(read - float(read_ms)) < 0.002
        assert abs(qt.net_saving(float(read_ms), 1.0, float(tc)) - float(net)) < 1e-12
        assert abs(qt.net_saving(float(saved_mib) * 2**20, float(tbps) * 1e9, float(tc)) - float(net)) < 0.002
    fa, sa, fb, sb, cross = _f(g["fits"][0])
    assert abs(qt.linear_crossover(fa, sa, fb, sb) - cross) < 1.0
    for L, a, b in g["fit_at"]:
        assert abs(fa + sa * float(L) - float(a)) < 0.005
        assert abs(fb + sb * float(L) - float(b)) < 0.005


def _exact_checks(fmt, x, codes, scales):
    """Rational checks of one array of groups; True when all hold."""
    qmax = qt.FORMATS[fmt][1]
    xs = np.asarray(x, dtype=np.float32).reshape(-1, 32)
    cs = codes.reshape(-1, 32)
    ss = scales.reshape(-1).view(np.float16)
    for row, crow, s16 in zip(xs, cs, ss):
        amax = Fraction(float(np.abs(row).max()))
        want = min(amax / qmax, Fraction(qt.HALF_MAX))  # saturates at the largest finite half
        s = Fraction(float(s16))
        # the stored scale is a half nearest max|x| / qmax (within half an ulp of the
        # float32 quotient, which is itself within half a float32 ulp)
        ulp = Fraction(2) ** (int(np.floor(np.log2(float(s16)))) - 10) if s16 > 0 else Fraction(2) ** -24
        if not abs(s - want) <= ulp / 2 + want * Fraction(1, 2**23):
            return False
        for xv, c in zip(row, crow):
            if s == 0:
                if c != 0:
                    return False
                continue
            r = Fraction(float(xv)) / s
            if abs(c) > qmax:
                return False
            if abs(r) <= qmax:
                # nearest integer, up to the float32 rounding of the quotient near a tie
                if abs(Fraction(int(c)) - r) > Fraction(1, 2) + abs(r) * Fraction(1, 2**23):
                    return False
            elif c != (qmax if r > 0 else -qmax):
                return False
    return True


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_codes_are_nearest_integers_of_the_scaled_values(fmt):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    x[3, :32] = 0.0                  # an all-zero group
    x[4, 5] = 1e6                    # one dominant value
    codes, scales = qt.quantize(x, fmt)
    assert codes.shape == x.shape and scales.shape == (40, 2)
    assert _exact_checks(fmt, x, codes, scales)
    # the largest magnitude of every group maps to a code of magnitude qmax or qmax - 1
    qmax = qt.FORMATS[fmt][1]
    g = codes.reshape(-1, 32).astype(int)
    nz = np.abs(x.reshape(-1, 32)).max(axis=1) > 0
    assert np.all(np.abs(g[nz]).max(axis=1) >= qmax - 1)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_values_on_the_code_grid_round_trip_exactly(fmt):
    qmax = qt.FORMATS[fmt][1]
    rng = np.random.default_rng(22)
    k = rng.integers(-qmax, qmax + 1, size=(16, 32))
    k[:, 0] = qmax                   # pins max|x| = qmax * step
    step = 2.0 ** rng.integers(-12, 4, size=(16, 1))
    x = (k * step).astype(np.float32)
    codes, scales = qt.quantize(x, fmt)
    assert np.array_equal(codes.astype(int), k)
    assert np.array_equal(qt.dequantize(codes, scales), x.astype(np.float64))


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_round_trip_error_is_at_most_half_a_step(fmt):
    rng = np.random.default_rng(23)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    codes, scales = qt.quantize(x, fmt)
    back = qt.dequantize(codes, scales)
    step = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=-1)
    assert np.all(np.abs(back - x) <= 0.5 * step * (1 + 2**-10) + 1e-30)


def test_q4_packing_round_trips_and_puts_the_even_value_low():
    rng = np.random.default_rng(24)
    c = rng.integers(-7, 8, size=(5, 64)).astype(np.int8)
    p = qt.pack_q4(c)
    assert p.shape == (5, 32)
    assert np.array_equal(qt.unpack_q4(p), c)
    assert qt.pack_q4(np.array([[-7, 7]], np.int8))[0, 0] == 0xF1


def _mutants():
    def scale_by_qmax_plus_one(x, fmt):
        qmax = qt.FORMATS[fmt][1]
        saved = qt.FORMATS[fmt]
        qt.FORMATS[fmt] = (saved[0], qmax + 1)
        try:
            codes, scales = qt.quantize(x, fmt)
        finally:
            qt.FORMATS[fmt] = saved
        return np.clip(codes, -qmax, qmax).astype(np.int8), scales

    def truncating(x, fmt):
        qmax = qt.FORMATS[fmt][1]
        x = np.asarray(x, np.float32)
        g = x.reshape(x.shape[:-1] + (-1, 32))
        s16 = (np.abs(g).max(axis=-1) / np.float32(qmax)).astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = g / s16.astype(np.float32)[..., None]
        c = np.where(s16[..., None] > 0, np.trunc(r), 0)
        return np.clip(c, -qmax, qmax).astype(np.int8).reshape(x.shape), s16.view(np.uint16)

    def unrounded_scale(x, fmt):
        # codes from the float32 scale, the half stored afterwards
        qmax = qt.FORMATS[fmt][1]
        x = np.asarray(x, np.float32)
        g = x.reshape(x.shape[:-1] + (-1, 32))
        s32 = np.abs(g).max(axis=-1) / np.float32(qmax)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = g / s32[..., None]
        c = np.where(s32[..., None] > 0, np.rint(r), 0)
        return np.clip(c, -qmax, qmax).astype(np.int8).reshape(x.shape), s32.astype(np.float16).view(np.uint16)

    def group_of_16(x, fmt):
        qmax = qt.FORMATS[fmt][1]
        x = np.asarray(x, np.float32)
        g = x.reshape(x.shape[:-1] + (-1, 16))
        s16 = (np.abs(g).max(axis=-1) / np.float32(qmax)).astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = g / s16.astype(np.float32)[..., None]
        c = np.where(s16[..., None] > 0, np.rint(r), 0)
        return (np.clip(c, -qmax, qmax).astype(np.int8).reshape(x.shape),
                s16.reshape(x.shape[:-1] + (-1, 2))[..., 0].view(np.uint16))

    return [scale_by_qmax_plus_one, truncating, unrounded_scale, group_of_16]


def _pins_hold(fn):
    ok = True
    for fmt in ("q8_0", "q4_0"):
        rng = np.random.default_rng(25)
        x = (rng.standard_normal((24, 64)) * np.exp(rng.uniform(-4, 4, (24, 1)))).astype(np.float32)
        codes, scales = fn(x, fmt)
        ok &= _exact_checks(fmt, x, codes, scales)
        qmax = qt.FORMATS[fmt][1]
        k = rng.integers(-qmax, qmax + 1, size=(8, 32)); k[:, 0] = qmax
        xg = (k * 2.0 ** rng.integers(-8, 4, size=(8, 1))).astype(np.float32)
        c2, s2 = fn(xg, fmt)
        ok &= np.array_equal(c2.astype(int), k)
    return ok


def test_oracle_passes_its_own_pins():
    assert _pins_hold(qt.quantize)


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    assert not _pins_hold(mutant)


def test_quantised_replay_gathers_the_dequantised_rows():
    """A quantised pool replayed through shuffled tables returns, for every
    position, the dequantised quantisation of the token's generated row; a copy
    on write copies codes and scales."""
    from dataclasses import replace

    from oracle.attention import decode_attention
    from oracle.runner import OracleReplay
    from synth import draws, workloads

    for fmt in ("q8_0", "q4_0"):
        base = workloads.chunked_prompt((70, 33), chunk=40)
        wl = replace(base, kv_format=fmt, ops=base.ops + [("fork", 0, 5), ("append", (5,), (1,)),
                                                            ("decode", (0, 1, 5))])
        ref = OracleReplay(wl).run()
        dec = ref.decodes[0]
        for i, s in enumerate((0, 1)):
            n = dec["lengths"][i]
            k, v = ref.gather_f64(0, dec["tables"][i], n)
            pos = np.arange(n)
            kr = draws.bits_to_f64(draws.token_rows(wl.seed, draws.TAG_K, 0, s, pos, wl.num_kv_heads,
                                                    wl.head_dim, wl.dtype), wl.dtype)
            vr = draws.bits_to_f64(draws.token_rows(wl.seed, draws.TAG_V, 0, s, pos, wl.num_kv_heads,
                                                    wl.head_dim, wl.dtype), wl.dtype)
            assert np.array_equal(k, qt.dequantize(*qt.quantize(kr, fmt)))
            assert np.array_equal(v, qt.dequantize(*qt.quantize(vr, fmt)))
            q = draws.bits_to_f64(ref.query_bits(0, 0), wl.dtype)[i]
            assert np.allclose(ref.attention(0, 0, rows=[i])[0], decode_attention(q, k, v), rtol=0, atol=1e-13)
        # the fork shares sequence 0's blocks up to the copied one
        k5, _ = ref.gather_f64(0, dec["tables"][2], 70)
        k0, _ = ref.gather_f64(0, dec["tables"][0], 70)
        assert np.array_equal(k5, k0)
