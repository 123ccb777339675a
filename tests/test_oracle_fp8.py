"""Pins of the FP8 embedding oracle: the E4M3 code table at known values, rounding ties to the
even code, code round trips, the per-row power-of-two exponent at its boundaries, the error
bound of the quantised rows, and exactness of the dequantised rows in bf16."""
import numpy as np

from denoise_step_sampler_amd import synth
from oracle import fp8


def test_code_table_known_values():
    v = fp8.e4m3_value(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8, 0x00, 0x80, 0x3C, 0x07],
                                np.uint8))
    assert list(v[:5]) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0]
    assert v[5] == 0.0 and v[6] == 0.0
    assert v[7] == 1.5 and v[8] == 7 * 2.0 ** -9
    assert np.isnan(fp8.e4m3_value(np.array([0x7F, 0xFF], np.uint8))).all()
    finite = fp8.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.nanmax(finite) == 448.0 and np.sum(np.isnan(finite)) == 2


def test_rounding_ties_and_round_trip():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code wins
    assert fp8.e4m3_round(np.array([1.0625]))[0] == 0x38
    assert fp8.e4m3_round(np.array([1.1875]))[0] == 0x3A       # between 0x39 and 0x3A
    assert fp8.e4m3_round(np.array([1.0626]))[0] == 0x39
    assert fp8.e4m3_round(np.array([-3.0 * 2.0 ** -10]))[0] == 0x82   # 1.5 quanta -> 2
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(fp8.e4m3_round(fp8.e4m3_value(codes)), codes)


def test_row_exponent_boundaries():
    a = np.array([448.0, 448.0000001, 224.0, 224.0000001, 1.0, 0.0, 448.0 * 2.0 ** -20,
                  2.0 ** -120])
    assert list(fp8.row_exponent(a)) == [0, 1, -1, 0, -8, -117, -20, -117]


def test_quantized_rows_error_and_bf16_exactness():
    E = synth.make_embedding(300, 64, seed=2)
    Ef = synth.bf16_to_f32(E).astype(np.float64)
    Ef[7] = 0.0
    Ef[8] *= 1e-30
    Ef[9] *= 2.0 ** -140          # below the exponent floor: coarser codes, still exact
    q, k = fp8.quantize_rows(Ef)
    D = fp8.dequantize_rows(q, k)
    amax = np.max(np.abs(Ef), axis=1)
    for v in range(300):
        if amax[v] == 0:
            assert np.all(D[v] == 0)
            continue
        if k[v] == fp8.K_MIN:
            assert amax[v] <= 448.0 * 2.0 ** k[v]
            continue
        # the row's largest entry lands in (224, 448] times the row scale (its code in
        # [224, 448]: values just above 224 round down to it)
        assert 224.0 < amax[v] / 2.0 ** k[v] <= 448.0
        top = np.abs(fp8.e4m3_value(q[v])).max()
        assert 224.0 <= top <= 448.0
        # error at most half a quantum of the E4M3 grid at each entry's magnitude
        big = np.abs(Ef[v]) >= 2.0 ** -6 * 2.0 ** k[v]
        rel = np.abs(D[v] - Ef[v])[big] / np.abs(Ef[v])[big]
        assert np.all(rel <= 2.0 ** -4 + 1e-15)
        assert np.all(np.abs(D[v] - Ef[v])[~big] <= 2.0 ** -10 * 2.0 ** k[v] + 1e-300)
    # dequantised values are bf16 numbers
    f32 = D.astype(np.float32)
    assert np.array_equal(synth.bf16_to_f32(synth.round_to_bf16(f32)), f32)
    assert np.array_equal(f32.astype(np.float64), D)


def test_dynamic_activation_rows_by_hand():
    """A hidden-state row quantised at run time: max |h| = 3 gives k = -7 (448 2^-8 = 1.75 < 3
    <= 3.5 = 448 2^-7); 3 * 2^7 = 384 = 1.5 2^8 -> 0x7C, -1 * 2^7 -> 0xF0, bf16(0.3) =
    0.30078125 -> 38.5 -> 40 = 1.25 2^5 -> 0x62 (dequantised 0.3125), 0 -> 0x00; a zero row
    takes the floor -117 and zero codes."""
    row = np.zeros((2, 8), np.float32)
    row[0, :4] = [3.0, -1.0, 0.3, 0.0]
    bits = synth.round_to_bf16(row)
    codes, k, hq = fp8.activation_rows(bits)
    assert list(k) == [-7, -117]
    assert list(codes[0, :4]) == [0x7C, 0xF0, 0x62, 0x00] and not codes[1].any()
    assert list(synth.bf16_to_f32(hq)[0, :4]) == [3.0, -1.0, 0.3125, 0.0]
    assert not synth.bf16_to_f32(hq)[1].any()
