"""Pins of the FP8 (OCP E4M3) KV-cache oracle (oracle/kv_fp8.py).

The format is pinned against torch's float8_e4m3fn on the CPU (a library
implementation of the same OCP format): all 256 codes decode to the same
values, and every in-range value -- representable values, midpoints between
neighbours (the ties), subnormals, random values -- encodes to the same code.
Saturation above 448 is this build's reading (torch gives NaN there) and is
pinned by itself.  The scale direction is pinned by exact round trips, and the
FP8 decode reduces to the plain attention oracle on the values the codes
stand for.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import kv_fp8


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn) \
        .float().numpy().astype(np.float64)


ALL = np.arange(256, dtype=np.uint8)


def test_decode_table_matches_torch_and_the_format():
    ours, ref = kv_fp8.decode_codes(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    named = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in named.items():
        assert kv_fp8.decode_codes([c])[0] == v, hex(c)
    assert np.isnan(kv_fp8.decode_codes([0x7F, 0xFF])).all()
    assert np.isnan(ours).sum() == 2                      # no infinities, two NaNs


def test_encode_matches_torch_on_representable_values_and_ties():
    pos = kv_fp8.decode_codes(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2                       # exact in float32
    quarter = pos[:-1] + (pos[1:] - pos[:-1]) / 4
    xs = np.concatenate([pos, mids, quarter, -pos, -mids, -quarter]).astype(np.float32)
    assert np.array_equal(kv_fp8.encode_values(xs), torch_encode(xs))


def test_encode_matches_torch_on_random_in_range_values():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.uniform(-464, 464, 20000), rng.standard_normal(20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),         # subnormal range
        np.exp2(rng.uniform(-12, 8.85, 20000)) * rng.choice([-1, 1], 20000)]).astype(np.float32)
    xs = xs[np.abs(xs) < 464]
    assert np.array_equal(kv_fp8.encode_values(xs), torch_encode(xs))


def test_saturation_nan_and_signed_zero():
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf], dtype=np.float32)
    assert (kv_fp8.encode_values(big) == 0x7E).all()
    assert (kv_fp8.encode_values(-big) == 0xFE).all()
    assert kv_fp8.encode_values([np.nan])[0] == 0x7F
    assert kv_fp8.encode_values([-0.0])[0] == 0x80
    assert kv_fp8.encode_values([-2.0 ** -11])[0] == 0x80  # rounds to zero, keeps the sign


def test_every_finite_code_round_trips_and_encoding_is_monotone():
    finite = ALL[~np.isnan(kv_fp8.decode_codes(ALL))]
    assert np.array_equal(kv_fp8.encode_values(kv_fp8.decode_codes(finite)), finite)
    x = np.sort(np.random.default_rng(1).uniform(0, 500, 50000)).astype(np.float32)
    assert (np.diff(kv_fp8.encode_values(x).astype(np.int64)) >= 0).all()


@pytest.mark.parametrize("scale", [1.0, 0.5, 2.0 ** -7, 8.0])
def test_scale_divides_before_encoding_and_multiplies_after(scale):
    finite = ALL[~np.isnan(kv_fp8.decode_codes(ALL))]
    x = (kv_fp8.decode_codes(finite) * scale).astype(np.float32)   # power-of-two scale: exact
    assert np.array_equal(kv_fp8.quantize(x, scale), finite)
    assert np.array_equal(kv_fp8.values(finite, scale), kv_fp8.decode_codes(finite) * scale)


def test_decode_reduces_to_plain_attention_on_the_values():
    rng = np.random.default_rng(2)
    S, hq, hkv, d, nb = 3, 4, 2, 64, 12
    k_codes = rng.integers(0, 256, (nb, hkv, 16, d), dtype=np.uint8)
    v_codes = rng.integers(0, 256, (nb, hkv, 16, d), dtype=np.uint8)
    for c in (k_codes, v_codes):                          # no NaN codes, magnitudes up to 448
        c[(c & 0x7F) == 0x7F] = 0x3C
    tables = np.array([[3, 7, 1], [0, 2, -1], [11, -1, -1]], dtype=np.int32)
    lens = np.array([40, 17, 5], dtype=np.int32)
    q = rng.standard_normal((S, hq, d)).astype(np.float32)
    ks, vs = 0.03125, 0.5
    got = kv_fp8.decode(q, k_codes, v_codes, tables, lens, np.float32(0.125), ks, vs, "f32")
    kp = (kv_fp8.decode_codes(k_codes) * ks).astype(np.float32)   # exact: few significant bits
    vp = (kv_fp8.decode_codes(v_codes) * vs).astype(np.float32)
    want = oracle.decode(q, kp, vp, tables, lens, np.float32(0.125), "f32")
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


def _prefill_case(seed):
    rng = np.random.default_rng(seed)
    hq, hkv, d, nb = 4, 2, 64, 16
    k_codes = rng.integers(0, 256, (nb, hkv, 16, d), dtype=np.uint8)
    v_codes = rng.integers(0, 256, (nb, hkv, 16, d), dtype=np.uint8)
    for c in (k_codes, v_codes):                          # no NaN codes
        c[(c & 0x7F) == 0x7F] = 0x3C
    tables = np.array([[3, 7, 1, 9], [0, 2, -1, -1], [11, 12, 13, -1]], dtype=np.int32)
    lens = np.array([50, 17, 40], dtype=np.int32)        # chunks of 7, 17 and 1 new tokens
    qsl = np.array([0, 7, 24, 25], dtype=np.int32)
    q = rng.standard_normal((25, hq, d)).astype(np.float32)
    return q, k_codes, v_codes, tables, qsl, lens


def test_prefill_reduces_to_plain_prefill_on_the_values():
    """Power-of-two scales keep the dequantised values exact in fp32, so the FP8
    prefill must equal the plain prefill oracle on those values."""
    q, kc, vc, tables, qsl, lens = _prefill_case(5)
    ks, vs, scale = 0.03125, 0.5, np.float32(0.125)
    got = kv_fp8.prefill(q, kc, vc, tables, qsl, lens, scale, ks, vs, "f32")
    kp = (kv_fp8.decode_codes(kc) * ks).astype(np.float32)
    vp = (kv_fp8.decode_codes(vc) * vs).astype(np.float32)
    want = oracle.prefill(q, kp, vp, tables, qsl, lens, scale, "f32")
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    # a planted swap of the two scales is a different result
    swapped = kv_fp8.prefill(q, kc, vc, tables, qsl, lens, scale, vs, ks, "f32")
    assert not np.allclose(swapped, want, rtol=1e-6, atol=1e-6)


def test_prefill_one_token_chunk_is_decode():
    """The last query of a chunk sees the whole context: a one-token chunk is
    the FP8 decode of that token (xdnf.cn article, section 六.4)."""
    q, kc, vc, tables, qsl, lens = _prefill_case(6)
    got = kv_fp8.prefill(q, kc, vc, tables, qsl, lens, np.float32(0.125), 0.07, 0.11, "f32")
    last = np.array([qsl[1] - 1, qsl[2] - 1, qsl[3] - 1])
    want = kv_fp8.decode(q[last], kc, vc, tables, lens, np.float32(0.125), 0.07, 0.11, "f32")
    np.testing.assert_allclose(got[last], want, rtol=1e-13, atol=1e-13)


def test_fp8_scatter_quantises_into_slots():
    rng = np.random.default_rng(4)
    nb, hkv, d = 6, 2, 64
    kp = np.zeros((nb, hkv, 16, d), dtype=np.uint8)
    vp = np.zeros_like(kp)
    key = rng.standard_normal((3, hkv, d)).astype(np.float32)
    val = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([17, -1, 95])
    k2, v2 = kv_fp8.reshape_and_cache(kp, vp, key, val, slots, "f32", 0.25, 0.0625)
    assert np.array_equal(k2[1, :, 1, :], kv_fp8.quantize(key[0], 0.25))
    assert np.array_equal(v2[5, :, 15, :], kv_fp8.quantize(val[2], 0.0625))
    k2[1, :, 1, :] = 0
    k2[5, :, 15, :] = 0
    assert not k2.any()


def test_planted_tie_away_encoder_is_caught():
    """Rounding ties away from zero instead of to even fails the torch pin."""
    pos = kv_fp8.decode_codes(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)

    def tie_away(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        lo = np.searchsorted(pos, np.minimum(np.abs(x), 448.0), side="right") - 1
        hi = np.minimum(lo + 1, len(pos) - 1)
        pick = (pos[hi] - np.abs(x)) <= (np.abs(x) - pos[lo])
        return np.where(pick, hi, lo).astype(np.uint8)
    assert not np.array_equal(tie_away(mids), torch_encode(mids))
