"""The one inexact step of the int8 decode kernels, checked on the CPU.

The decode, stream, flat and group kernels feed the int8 matrix cores with
each token quantised to q = round(x 2^sh) (nearest, ties to even), one power
of two per token: with max|x| in [2^(E-1), 2^E) the shift is sh = 22 - E, so
|x 2^sh| < 2^22, and q is split into three signed bytes l_0 + 2^8 l_1 +
2^16 l_2.  The kernels form q + 0x808080 as the fp32 bit pattern of
x 2^sh + 1.5 2^23 minus 0x4ABF7F80 (the product is exact, the addition
rounds to an integer) and read the bytes of that, each xor 0x80.

This file models that reading in numpy and checks, for every finite fp16
value as an element of a token of every possible maximum binade, that
  * |q| <= 2^22, so three signed bytes hold it,
  * the bytes reconstruct q exactly,
  * the element error |x - q 2^-sh| <= 2^(E-23) <= 2^-22 max|x|,
  * an all-zero token gives q = 0 (so y = 0 exactly).
The dual-scale variants quantise the fp32 products x_j h_k[j] the same way,
with E taken from the fp32 maximum; the same bound holds per copy.
The product's error bound follows: |y - y_exact| <= sum_k |a_k| sum_j
|dx_j| <= K max|a| n 2^-22 max|x| before the fp16 output rounding.
"""
import numpy as np

FP16_FINITE = np.arange(0, 0x7C00, dtype=np.uint16)   # all non-negative finite fp16 patterns


def shift_for_max_fp16(mx_bits):
    """sh from the fp16 bit pattern of max|x| (biased exponent e, 0 for
    subnormals and zero): |x| < 2^E with E = max(e, 1) - 14, sh = 22 - E."""
    e = int(mx_bits) >> 10
    return 22 - (max(e, 1) - 14)


def quantise(x32, sh):
    """q + 0x808080 the way the kernels form it: the fp32 bit pattern of
    x 2^sh + 1.5 2^23, minus 0x4ABF7F80."""
    t = (np.asarray(x32, np.float32) * np.float32(2.0 ** sh)).astype(np.float32)   # exact
    t = (t + np.float32(12582912.0)).astype(np.float32)                            # rounds
    return t.view(np.uint32).astype(np.int64) - 0x4ABF7F80


def limbs(v):
    """Three signed bytes of v = q + 0x808080."""
    b = [((v >> (8 * i)) & 0xFF) ^ 0x80 for i in range(3)]
    return [np.where(x >= 128, x - 256, x) for x in b]


def test_every_fp16_value_in_every_binade():
    vals = FP16_FINITE.view(np.float16).astype(np.float32)
    signed = np.concatenate([vals, -vals])
    for mx_bits in range(0, 0x7C00, 0x400):          # the smallest pattern of every binade, and zero
        for top in (mx_bits, mx_bits | 0x3FF):       # its smallest and largest maximum
            mx = np.float32(np.uint16(top).view(np.float16))
            sh = shift_for_max_fp16(top)
            E = 22 - sh
            x = signed[np.abs(signed) <= mx]
            v = quantise(x, sh)
            q = v - 0x808080
            assert np.abs(q).max() <= 2 ** 22
            l0, l1, l2 = limbs(v)
            assert np.array_equal(l0 + 256 * l1 + 65536 * l2, q)
            err = np.abs(x.astype(np.float64) - q.astype(np.float64) * 2.0 ** -sh)
            assert err.max() <= 2.0 ** (E - 23)
            if mx > 0:
                assert err.max() <= 2.0 ** -22 * float(mx)
                assert mx < 2.0 ** E and (top < 0x400 or mx >= 2.0 ** (E - 1))
            # q = round(x 2^sh) to nearest, ties to even
            assert np.array_equal(q, np.rint(x.astype(np.float64) * 2.0 ** sh).astype(np.int64))


def test_zero_token_quantises_to_zero():
    sh = shift_for_max_fp16(0)
    x = np.array([0.0, -0.0] * 8, dtype=np.float32)
    assert (quantise(x, sh) - 0x808080 == 0).all()


def test_mixed_token_keeps_its_own_scale():
    """65504 next to 1e-3 values: the small ones fall below half a quantum
    (2^-7 at sh = 6) and become 0; their loss is within the bound."""
    x = np.array([65504.0, -65504.0, 1e-3, -2e-3, 3e-3], dtype=np.float16).astype(np.float32)
    mx_bits = int(np.abs(x).astype(np.float16).view(np.uint16).max())
    sh = shift_for_max_fp16(mx_bits)
    assert sh == 6
    q = quantise(x, sh) - 0x808080
    assert list(q) == [65504 * 64, -65504 * 64, 0, 0, 0]
    assert np.abs(x - q * 2.0 ** -sh).max() <= 2.0 ** -22 * 65504


def test_dual_products_bound():
    """x_j h_j is exact in fp32 (two binary16 factors); the shift comes from
    the fp32 maximum: max < 2^(e8 - 126) with e8 its biased exponent, sh =
    148 - e8.  Extremes: 65504^2 and 2^-48 (the smallest product of two
    subnormals)."""
    rng = np.random.default_rng(5)
    for scale in (65504.0, 1.0, 2.0 ** -12, 2.0 ** -24):
        xv = (rng.uniform(-1, 1, 4096) * scale).astype(np.float16).astype(np.float32)
        hv = (rng.uniform(-1, 1, 4096) * scale).astype(np.float16).astype(np.float32)
        p = (xv * hv).astype(np.float32)
        assert np.array_equal(p.astype(np.float64), xv.astype(np.float64) * hv.astype(np.float64))
        mx = np.abs(p).max()
        if mx == 0:
            continue
        e8 = int(np.float32(mx).view(np.uint32)) >> 23
        sh = 148 - e8
        E = 22 - sh
        assert mx < 2.0 ** E
        q = quantise(p, sh) - 0x808080
        assert np.abs(q).max() <= 2 ** 22
        assert np.abs(p.astype(np.float64) - q * 2.0 ** -sh).max() <= 2.0 ** (E - 23)
