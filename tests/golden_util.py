"""Reading the hand-worked examples of tests/golden/worked_examples.json."""

import numpy as np


def f32_from_hex(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def golden_arrays(ex):
    """(W, X, q, xq) of a worked example: dense lists, or the shape and the non-zero
    entries [row, col, value] (values may be fp32 bit patterns in hex)."""
    def dense(key, shape, dtype):
        if key in ex:
            return np.array(ex[key], dtype=dtype)
        out = np.zeros(shape, dtype=dtype)
        for r, c, v in ex[key + "_entries"]:
            out[r, c] = f32_from_hex(v) if isinstance(v, str) else v
        return out
    w = dense("W", ex.get("shape"), np.float32)
    x = dense("X", ex.get("X_shape"), np.float32)
    return w, x, dense("q", w.shape, np.int8), dense("xq", x.shape, np.int8)


def hex_bits(rows, dtype=np.uint32):
    """Nested lists of hex strings -> an array of bit patterns."""
    return np.array([[int(h, 16) for h in r] for r in rows], dtype=dtype)


def norm_example_arrays(ex):
    """(v [1, K], w [K]) of a hand-worked norm example."""
    k = ex["K"]
    v = np.zeros((1, k), np.float32)
    for i, val in ex["v_entries"]:
        v[0, i] = val
    w = np.full(k, ex["w_default"], np.float32)
    for i, val in ex["w_entries"]:
        w[i] = val
    return v, w
