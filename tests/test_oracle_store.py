"""Pins for the oracle's store path (quantisation, row layout, slab mean)."""
import numpy as np

from oracle.codecs import e4m3_decode
from oracle.layout import RowLayout
from oracle.store import quantize_tokens, read_kv, slab_entry, write_tokens
from workload import gen, get_workload


def _grid_tokens(n, H=4, d=128, seed=0):
    rng = np.random.default_rng(seed)
    return (np.clip(np.rint(rng.standard_normal((n, H, d)) * 16), -64, 64) / 16).astype(np.float32)


def test_fp8_relative_error_bound():
    """Dequantised values are within half an e4m3 ulp: 2^-4 relative in the
    normal range, 2^-10 * scale absolute in the subnormal range."""
    x = _grid_tokens(64)
    codes, scale = quantize_tokens(x)
    xr = e4m3_decode(codes).astype(np.float64) * scale[:, None, None]
    err = np.abs(xr - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))


def test_amax_element_maps_to_448():
    x = _grid_tokens(64, seed=1)
    codes, scale = quantize_tokens(x)
    flat = np.abs(x.reshape(64, -1))
    arg = flat.argmax(axis=1)
    c = codes.reshape(64, -1)[np.arange(64), arg] & 0x7F
    assert np.all(c == 0x7E)


def test_zero_token_scale_one():
    x = np.zeros((2, 4, 128), dtype=np.float32)
    codes, scale = quantize_tokens(x)
    assert np.all(scale == 1.0) and np.all(codes == 0)


def test_scale_is_fp32_division():
    x = _grid_tokens(8, seed=2)
    _, scale = quantize_tokens(x)
    amax = np.abs(x.reshape(8, -1)).max(axis=1)
    # the scale times 448 recovers amax to within one fp32 ulp
    assert np.all(np.abs(scale.astype(np.float64) * 448 - amax) <= np.spacing(amax.astype(np.float32)))


def test_row_layout_sizes_match_survey_shapes():
    lay = RowLayout(12, 4, 64, 128, True)
    assert lay.layer_bytes == 66048 and lay.row_bytes == 792576
    assert RowLayout(1, 1, 16, 128, False).row_bytes == 8192


def test_write_read_roundtrip_positions():
    """bf16 rows store values verbatim: every (head, token, dim) lands where
    read_kv finds it."""
    lay = RowLayout(2, 2, 8, 128, False)
    row = np.zeros(lay.row_bytes, dtype=np.uint8)
    k = (np.arange(8 * 2 * 128).reshape(8, 2, 128) % 251 - 125).astype(np.float32)
    v = -k
    write_tokens(row, lay, 1, 0, k, v)
    kr, vr = read_kv(row, lay, 1)
    assert np.array_equal(kr.transpose(1, 0, 2), k) and np.array_equal(vr.transpose(1, 0, 2), v)
    k0, _ = read_kv(row, lay, 0)
    assert not np.any(k0)


def test_fresh_page_write_zero_fills_tail():
    lay = RowLayout(1, 4, 64, 128, True)
    row = np.full(lay.row_bytes, 0xAB, dtype=np.uint8)
    x = _grid_tokens(10, seed=3)
    write_tokens(row, lay, 0, 0, x, x)
    k, _ = read_kv(row, lay, 0)
    assert not np.any(k[:, 10:])
    # an append after offset 0 does not touch other positions
    row2 = row.copy()
    write_tokens(row2, lay, 0, 10, x[:3], x[:3])
    k2, _ = read_kv(row2, lay, 0)
    assert np.array_equal(k2[:, :10], k[:, :10]) and not np.any(k2[:, 13:])


def test_slab_is_bf16_of_numpy_mean():
    x = _grid_tokens(64, seed=4)
    ref = x.astype(np.float64).mean(axis=0)      # exact on the 2^-4 grid
    got = slab_entry(x)
    # bf16 of the mean: relative error <= 2^-9
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-12)
    # the mean of a page of 64 grid keys is a multiple of 2^-10
    assert np.all(np.mod(got.astype(np.float64) * 1024, 1) == 0)


def test_generator_values_on_grid_and_bf16_exact():
    wl = get_workload("c2")
    k = gen.kv_page(wl, gen.KIND_K, 3, 0, 17)
    assert k.shape == (64, 4, 128)
    assert np.all(np.mod(k * 16, 1) == 0) and np.abs(k).max() <= 4
    gen.to_bf16_bits(k)
    q = gen.prefill_queries(get_workload("c5"), 0, 5, 70)
    assert q.shape == (70, 32, 128) and np.all(np.mod(q * 32, 1) == 0)


def test_fp8_value_codes_are_stored_transposed():
    """fp8 V codes of token t, head h, dim d sit at [h][d][t] of the layer's V
    block (K codes at [h][t][d])."""
    lay = RowLayout(1, 2, 8, 128, True)
    row = np.zeros(lay.row_bytes, dtype=np.uint8)
    k = np.zeros((8, 2, 128), dtype=np.float32)
    v = np.zeros((8, 2, 128), dtype=np.float32)
    v[5, 1, 77] = 3.0          # one nonzero value: its token's amax -> code 0x7E
    k[2, 0, 9] = -2.0
    write_tokens(row, lay, 0, 0, k, v)
    vb = row[lay.v_off(0):lay.v_off(0) + lay.code_bytes]
    kb = row[lay.k_off(0):lay.k_off(0) + lay.code_bytes]
    assert np.flatnonzero(vb).tolist() == [(1 * 128 + 77) * 8 + 5] and vb[(1 * 128 + 77) * 8 + 5] == 0x7E
    assert np.flatnonzero(kb).tolist() == [(0 * 8 + 2) * 128 + 9] and kb[(0 * 8 + 2) * 128 + 9] == 0xFE
    kr, vr = read_kv(row, lay, 0)
    # 448 * fp32(amax / 448) recovers amax to one fp32 rounding of the scale
    assert abs(vr[1, 5, 77] - 3.0) < 1e-6 and abs(kr[0, 2, 9] + 2.0) < 1e-6
    assert np.count_nonzero(vr) == 1 and np.count_nonzero(kr) == 1


# ---------------------------------------------------------------- golden tokens --
import json as _json
import os as _os

_QGOLD = _os.path.join(_os.path.dirname(__file__), "golden", "quant_tokens.json")


def _golden_tokens():
    doc = _json.load(open(_QGOLD))
    toks = []
    for t in doc["tokens"]:
        xb = np.array([int(b, 16) for b in t["x_bf16_bits"]], dtype=np.uint32) << 16
        x = xb.view(np.float32).reshape(1, 1, -1)
        toks.append((x, int(t["scale_f32_bits"], 16), [int(c, 16) for c in t["codes"]],
                     int(t["reciprocal_form_scale_f32_bits"], 16), [int(c, 16) for c in t["reciprocal_form_codes"]]))
    return toks


def _quant_matches_golden(quant_fn):
    """True when `quant_fn` reproduces every golden token's scale bits and codes."""
    for x, sbits, codes, _, _ in _golden_tokens():
        c, s = quant_fn(x)
        if int(np.asarray(s, dtype=np.float32).view(np.uint32)[0]) != sbits:
            return False
        if [int(v) for v in np.asarray(c).reshape(-1)] != codes:
            return False
    return True


def _quant_reciprocal_form(x):
    """A plausible wrong quantiser: scale = amax * fp32(1/448) and codes from
    x * fp32(1/scale) -- two roundings where the definition has one."""
    from oracle.codecs import e4m3_encode
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    amax = np.abs(x.reshape(n, -1)).max(axis=1).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1), amax * (np.float32(1) / np.float32(448))).astype(np.float32)
    inv = (np.float32(1) / scale).astype(np.float32)
    return e4m3_encode((x * inv[:, None, None]).astype(np.float32)), scale


def test_quantiser_matches_golden_tokens():
    """Scale bits and codes of hand-picked tokens, computed with exact
    rationals from the definition (tests/golden/make_quant_golden.py)."""
    assert _quant_matches_golden(quantize_tokens)


def test_golden_tokens_separate_the_reciprocal_form():
    """The tokens pin the single-rounding definition: the reciprocal-multiply
    quantiser gets different scales and codes on them (checked both against
    the generator's own record of that form and by running it)."""
    toks = _golden_tokens()
    assert any(t[1] != t[3] for t in toks) and any(t[2] != t[4] for t in toks)
    for x, _, _, rs, rc in toks:
        c, s = _quant_reciprocal_form(x)
        assert int(s.view(np.uint32)[0]) == rs and [int(v) for v in c.reshape(-1)] == rc
    assert not _quant_matches_golden(_quant_reciprocal_form)


def test_slab_mean_off_grid_is_one_rounding_of_the_exact_sum():
    """General bf16 keys (not on a grid): the slab entry is bf16(fp32(exact
    sum) / n); the exact sum is taken with Python fractions."""
    from fractions import Fraction
    from oracle.codecs import bf16_round
    rng = np.random.default_rng(11)
    k = bf16_round(rng.standard_normal((64, 2, 16)).astype(np.float32))
    got = slab_entry(k)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_quant_golden", _os.path.join(_os.path.dirname(__file__), "golden", "make_quant_golden.py"))
    exact_fp = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(exact_fp)
    for h in range(2):
        for d in range(16):
            exact = sum(Fraction(float(v)) for v in k[:, h, d])
            f32 = np.uint32(exact_fp.f32_bits(exact)).view(np.float32)      # one RNE rounding to fp32
            mean = np.uint32(exact_fp.f32_bits(Fraction(float(f32)) / 64)).view(np.float32)
            exp = bf16_round(np.array([mean], dtype=np.float32))[0]
            assert got[h, d] == exp


def test_slab_certificate_trips_on_keys_too_wide_for_fp64():
    """The tier refuses to store a page whose fp64 key sums it cannot prove
    exact (a key of 2^100 beside one of 2^-100 in the same feature)."""
    import pytest
    from oracle.engine import OracleTier, SlabCertificateError
    t = OracleTier(num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16, fp8=False,
                   num_logical_pages=4, num_slots=4)
    bt = np.arange(4, dtype=np.int32)[None, :]
    t.ensure_write_pages([(0, 0, 16)], bt, [0])
    k = np.zeros((16, 1, 128), dtype=np.float32)
    k[0, 0, 0] = 2.0 ** 100
    k[1, 0, 0] = 2.0 ** -100
    with pytest.raises(SlabCertificateError):
        t.store(0, [(0, 0, 16)], k, k, bt)
    # N(0,1) keys in bf16 pass
    rng = np.random.default_rng(3)
    from oracle.codecs import bf16_round
    k = bf16_round(rng.standard_normal((16, 1, 128)).astype(np.float32))
    t.store(0, [(0, 0, 16)], k, k, bt)
