"""Pins of the oracle's OCP e4m3 functions (decode, encode, scaled
quantization, the fp8 cache and attention)."""
import numpy as np
import pytest

from hybrid_kv_cache_amd import workloads as W
from oracle import forcing_kv as O


def test_decode_spec_values():
    d = O.e4m3_decode
    assert d(np.uint8(0x7E)) == 448.0 and d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x38)) == 1.0 and d(np.uint8(0x40)) == 2.0 and d(np.uint8(0x3C)) == 1.5
    assert d(np.uint8(0x08)) == 2.0 ** -6          # smallest normal
    assert d(np.uint8(0x01)) == 2.0 ** -9          # smallest subnormal
    assert d(np.uint8(0x07)) == 7 * 2.0 ** -9      # largest subnormal
    assert np.isnan(d(np.uint8(0x7F))) and np.isnan(d(np.uint8(0xFF)))
    assert d(np.uint8(0x00)) == 0.0 and np.signbit(d(np.uint8(0x80)))


def test_codes_are_monotone_and_round_trip():
    c = np.arange(0x7F, dtype=np.uint8)                # non-negative finite codes
    v = O.e4m3_decode(c)
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(O.e4m3_encode(v.astype(np.float32)), c)
    assert np.array_equal(O.e4m3_encode(-v[1:].astype(np.float32)), c[1:] | 0x80)


def test_encode_nearest_even_and_saturation():
    v = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for i in range(0x7E):
        lo, hi = v[i], v[i + 1]
        mid = np.float32((lo + hi) / 2)                # exact in float32 here
        assert float(mid) == (lo + hi) / 2
        even = i if i % 2 == 0 else i + 1              # the even code wins a tie
        assert O.e4m3_encode(mid) == even
        assert O.e4m3_encode(np.float32(lo + (hi - lo) * 0.25)) == i
        assert O.e4m3_encode(np.float32(lo + (hi - lo) * 0.75)) == i + 1
    assert O.e4m3_encode(np.float32(1e6)) == 0x7E and O.e4m3_encode(np.float32(-500)) == 0xFE
    assert O.e4m3_encode(np.float32(2.0 ** -11)) == 0      # below half the smallest step


def test_brute_force_nearest_code():
    """Every random float32 maps to a nearest representable value (brute force
    over all 127 magnitudes)."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-9, 6, 4000))).astype(np.float32)
    mags = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    got = O.e4m3_decode(O.e4m3_encode(x))
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    best = np.min(np.abs(mags[None, :] - a[:, None]), axis=1)
    np.testing.assert_array_equal(np.abs(np.abs(got) - a), best)


def _bf16(x: float) -> np.ndarray:
    return W.round_to_bf16_bits(np.array([x], dtype=np.float32))


# (x, scale, code) worked out by hand from the e4m3 format: in the binade
# [2^E, 2^(E+1)) the step is 2^(E-3) and the code is (E + 7) << 3 | mantissa;
# below 2^-6 the step is 2^-9 (subnormals, exponent field 0).
HAND_CODES = [
    (3.0, 0.37, 0x50),        # 8.108.. -> [8, 16), step 1 -> 8: exponent 10, mantissa 0
    (-0.7, 0.37, 0xBF),       # bf16 -0.69921875 / 0.37 = -1.8897.. -> step 1/8 -> -1.875
    (100.0, 0.37, 0x78),      # 270.27.. -> [256, 512), step 32 -> 256: exponent 15
    (0.001, 1.0, 0x01),       # bf16 0.00099945.. = 0.5117 steps of 2^-9 -> 1 step
    (1000.0, 1.0, 0x7E),      # beyond the largest finite value: saturates to 448
    (2.0 ** -10, 1.0, 0x00),  # half a subnormal step: tie to the even code 0
    (3 * 2.0 ** -10, 1.0, 0x02),  # 1.5 subnormal steps: tie to the even code 2
]


@pytest.mark.parametrize("x,scale,code", HAND_CODES)
def test_quantize_hand_computed_codes(x, scale, code):
    assert int(O.quantize_e4m3(_bf16(x), scale)[0]) == code


def test_quantize_divides_in_float32():
    """x = 1.6953125 (bf16 0x3FD9) over the float32 scale 0x3FCC3C3C: the exact
    quotient is 1.0625 + 1.9e-8, just above the midpoint between 1.0 (0x38)
    and 1.125 (0x39), but the IEEE float32 quotient is exactly 1.0625, a tie
    that goes to the even code 0x38.  Dividing in a wider type gives 0x39."""
    x = np.array([0x3FD9], dtype=np.uint16)
    s = float(np.array([0x3FCC3C3C], dtype=np.uint32).view(np.float32)[0])
    assert float(np.float32(W.bf16_bits_to_f32(x)[0]) / np.float32(s)) == 1.0625
    assert int(O.quantize_e4m3(x, s)[0]) == 0x38


def _exact_fp8_case(seed=3, H=3, D=16, lens=(40, 70, 25), n_q=24):
    """Queries, keys and values that are e4m3 values times per-head powers of
    two, so that every quantization step is exact.  Each head's data include
    the largest finite magnitude (448) and the smallest subnormal (2^-9), so
    quantizing with another head's scale (2x or 4x off) saturates or rounds
    them away."""
    rng = np.random.default_rng(seed)
    q_s = np.array([2.0 ** -3, 2.0 ** 1, 2.0 ** -1])[:H]
    k_s = np.array([2.0 ** -4, 2.0 ** -6, 2.0 ** -2])[:H]
    v_s = np.array([2.0 ** 0, 2.0 ** -3, 2.0 ** 2])[:H]

    def codes(n):
        c = rng.integers(0, 0x7F, size=(n, D)).astype(np.uint8)   # finite magnitudes
        c |= (rng.integers(0, 2, size=(n, D)) << 7).astype(np.uint8)
        c[0, 0], c[-1, -1] = 0x7E, 0x01                           # 448 and 2^-9
        return c

    tok_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    k8 = np.concatenate([codes(n) for n in lens])
    v8 = np.concatenate([codes(n) for n in lens])
    # scale the random codes down so that the logits stay moderate
    qv = np.stack([O.e4m3_decode(codes(n_q)) * q_s[h] * 2.0 ** -8 for h in range(H)], axis=1)
    qb = W.round_to_bf16_bits(qv.astype(np.float32))
    assert np.array_equal(O.decode_bf16(qb), qv)                  # exact in bf16
    return qb, k8, v8, tok_off, q_s * 2.0 ** -8, k_s, v_s


def test_attend_fp8_exact_with_power_of_two_scales():
    """With every value an e4m3 value times its head's power-of-two scale, the
    fp8 attention must equal plain attention on those values (float64,
    1e-12): each head's q, k and v must be scaled by that head's own scale."""
    qb, k8, v8, tok_off, q_s, k_s, v_s = _exact_fp8_case()
    H = len(q_s)
    kv = np.empty(k8.shape)
    vv = np.empty(v8.shape)
    for h in range(H):
        lo, hi = tok_off[h], tok_off[h + 1]
        kv[lo:hi] = O.e4m3_decode(k8[lo:hi]) * k_s[h]
        vv[lo:hi] = O.e4m3_decode(v8[lo:hi]) * v_s[h]
    want = O.attend(O.decode_bf16(qb), kv, vv, tok_off)
    got = O.attend_fp8(qb, k8, v8, tok_off, q_s, k_s, v_s)
    assert np.abs(got - want).max() <= 1e-12
    # the pin has teeth: another head's scales give another result
    for perm in ([1, 2, 0], [2, 0, 1]):
        bad = O.attend_fp8(qb, k8, v8, tok_off, q_s[perm], k_s, v_s)
        assert np.abs(bad - want).max() > 1e-3
        bad = O.attend_fp8(qb, k8, v8, tok_off, q_s, k_s[perm], v_s)
        assert np.abs(bad - want).max() > 1e-3
        bad = O.attend_fp8(qb, k8, v8, tok_off, q_s, k_s, v_s[perm])
        assert np.abs(bad - want).max() > 1e-3


def test_compress_fp8_codes_exact_with_power_of_two_scales():
    """K and V of a layer made of e4m3 values times per-head powers of two:
    the cache codes decoded and multiplied by the head's scale give back the
    compacted bf16 rows exactly."""
    w = W.small_workload(tokens_per_frame=12, num_heads=3, hist_frames=6, head_dim=16, seed=9)
    inp = W.generate_layer(w)
    rng = np.random.default_rng(10)
    H, D = w.num_heads, w.head_dim
    k_s = np.array([2.0 ** -5, 2.0 ** -2, 2.0 ** 1])
    v_s = np.array([2.0 ** 0, 2.0 ** -7, 2.0 ** -3])
    kc = rng.integers(0, 0x7F, size=(w.n_win, H, D)).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(w.n_win, H, D)).astype(np.uint8)
    kc[0, :, 0], vc[0, :, 0] = 0x7E, 0x01
    kf = (O.e4m3_decode(kc) * k_s[None, :, None]).astype(np.float32)
    vf = (O.e4m3_decode(vc) * v_s[None, :, None]).astype(np.float32)
    k, v = W.round_to_bf16_bits(kf), W.round_to_bf16_bits(vf)
    assert np.array_equal(O.decode_bf16(k), kf.astype(np.float64))
    r = O.compress_fp8(inp.q, k, v, inp.head_role, inp.static_keep_mask, w.budget_m,
                       w.tokens_per_frame, w.hist_frames, w.cur_frames, w.query_stride,
                       k_s, v_s)
    for h in range(H):
        lo, hi = r["tok_off"][h], r["tok_off"][h + 1]
        assert np.array_equal(O.e4m3_decode(r["k8"][lo:hi]) * k_s[h], O.decode_bf16(r["k_c"][lo:hi]))
        assert np.array_equal(O.e4m3_decode(r["v8"][lo:hi]) * v_s[h], O.decode_bf16(r["v_c"][lo:hi]))


def test_fp8_attention_against_bf16_path():
    """With fine scales (codes use the full range) the fp8 attention stays
    close to the bf16 oracle: the quantization error bound of e4m3 (a relative
    step of 2^-3 at most, 2^-4 on average) over averaged outputs."""
    w = W.small_workload(tokens_per_frame=20, num_heads=3, hist_frames=6, seed=8)
    inp = W.generate_layer(w)
    T, Fh, Fc = w.tokens_per_frame, w.hist_frames, w.cur_frames
    amax = lambda a: np.abs(O.decode_bf16(a)).reshape(-1, w.num_heads, w.head_dim).max(axis=(0, 2))
    ks, vs, qs = amax(inp.k) / 448, amax(inp.v) / 448, amax(inp.q) / 448
    r = O.compress_fp8(inp.q, inp.k, inp.v, inp.head_role, inp.static_keep_mask, w.budget_m,
                       T, Fh, Fc, w.query_stride, ks, vs)
    ref = O.attend(inp.q, r["k_c"], r["v_c"], r["tok_off"])
    got = O.attend_fp8(inp.q, r["k8"], r["v8"], r["tok_off"], qs, ks, vs)
    assert np.abs(got - ref).max() < 0.1 and np.abs(got - ref).mean() < 0.01
    # exact scale 1 and values that are already codes: no error at all
    k1 = np.clip(np.round(O.decode_bf16(r["k_c"]) * 2) / 2, -4, 4)   # halves in [-4, 4]
    assert np.array_equal(O.e4m3_decode(O.quantize_e4m3(k1.astype(np.float32), 1.0)), k1)
