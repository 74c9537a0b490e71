"""The decode and act-quant kernels take an int8 code as the low byte of
RN32(t + 1.5 * 2^23), t = RN32(x * s), instead of clip(rne(t), -128, 127) (the
code of the per-token absmax quantisation: communeify.com page on BitNet b1.58
2B4T, quantisation details, 8-bit activations; onedollarvps.pages.dev BitNet
B1.58 guide, section 2, round and clip).  These CPU checks run the same float32
arithmetic in numpy (round to nearest, ties to even, like the GPU's default mode)
over every t a finite input can give, |t| <= 127 (1 + 2^-24), at and around
each half-integer, and over random quotients."""

import numpy as np

MAGIC = np.float32(12582912.0)   # 1.5 * 2^23


def low_byte_code(t):
    u = (t.astype(np.float32) + MAGIC).astype(np.float32)
    return (u.view(np.uint32) & 0xFF).astype(np.uint8).view(np.int8)


def reference_code(t):
    return np.clip(np.rint(t.astype(np.float32)), -128, 127).astype(np.int8)


def test_half_integers_and_neighbours():
    ks = np.arange(-128, 128, dtype=np.float32)
    centres = np.concatenate([ks, ks + np.float32(0.5)]).astype(np.float32)
    t = [centres]
    lo, hi = centres.copy(), centres.copy()
    for _ in range(64):                      # 64 floats either side of each centre
        lo = np.nextafter(lo, np.float32(-np.inf)).astype(np.float32)
        hi = np.nextafter(hi, np.float32(np.inf)).astype(np.float32)
        t += [lo, hi]
    t = np.concatenate(t)
    t = t[np.abs(t) <= np.float32(127.0) * np.float32(1 + 2.0 ** -23)]
    np.testing.assert_array_equal(low_byte_code(t), reference_code(t))


def test_signed_zero_and_tiny():
    t = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-38, -1e-38, 0.49999997, -0.49999997,
                  0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5, 127.0, -127.0],
                 dtype=np.float32)
    np.testing.assert_array_equal(low_byte_code(t), reference_code(t))


def test_random_quotients_with_token_scale():
    # t = RN32(x * RN32(127 / a*)) for rows whose absmax a* is the row's max |x|,
    # the largest |t| the kernels meet
    rng = np.random.Generator(np.random.PCG64(1234))
    for scale in (1e-30, 1e-6, 1.0, 3.0, 1e6, 1e30):
        x = (rng.standard_normal((64, 4096)) * scale).astype(np.float32)
        a = np.maximum(np.abs(x).max(axis=1), np.float32(1e-5)).astype(np.float32)
        s = (np.float32(127.0) / a).astype(np.float32)
        t = (x * s[:, None]).astype(np.float32)
        assert np.abs(t).max() <= np.float32(127.0) * np.float32(1 + 2.0 ** -23)
        np.testing.assert_array_equal(low_byte_code(t), reference_code(t))
