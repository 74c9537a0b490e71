"""C ABI checks that need no GPU: the library loads, exports every function the
public header declares, and rejects bad arguments before making any HIP call."""

import ctypes
import os
import re

import pytest

from ternary_weight_linear_bit_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet_mi355x.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x10002)    # 2-byte aligned only


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitnet_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        pytest.skip("libbitnet_mi355x.so not built")
    return N.lib()


def test_header_declares_expected_calls():
    names = header_functions()
    for want in ("bitnet_quantize_weights", "bitnet_quantize_acts", "bitnet_ternary_linear"):
        assert want in names


def test_library_exports_every_header_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in N.SIGNATURES, f"binding lacks {name}"


def test_status_strings_and_sizes(lib):
    for s in range(0, 8):
        assert lib.bitnet_status_string(s)
    assert lib.bitnet_packed_bytes(2560, 6912) == 2560 * 6912 // 4
    assert lib.bitnet_packed_bytes(3, 6) == 0
    assert lib.bitnet_packed_bytes(-1, 8) == 0
    assert lib.bitnet_quantize_weights_workspace_bytes(1, 4) == 16640   # 8 x 256 buckets + threshold


def test_quantize_weights_validation(lib):
    f = lib.bitnet_quantize_weights
    ws = lib.bitnet_quantize_weights_workspace_bytes(4, 8)
    assert f(None, 0, 4, 8, FAKE, FAKE, FAKE, ws, None) == ENULL
    assert f(FAKE, 0, 4, 8, None, FAKE, FAKE, ws, None) == ENULL
    assert f(FAKE, 9, 4, 8, FAKE, FAKE, FAKE, ws, None) == EDTYPE
    assert f(FAKE, 0, 0, 8, FAKE, FAKE, FAKE, ws, None) == ESHAPE
    assert f(FAKE, 0, 4, 6, FAKE, FAKE, FAKE, ws, None) == ESHAPE
    assert f(FAKE, 0, 4, 0, FAKE, FAKE, FAKE, ws, None) == ESHAPE
    assert f(FAKE, 0, 1 << 20, 1 << 18, FAKE, FAKE, FAKE, ws, None) == ESHAPE  # N*K = 2^38
    assert f(FAKE, 0, 4, 8, FAKE, FAKE, None, ws, None) == EWS
    assert f(FAKE, 0, 4, 8, FAKE, FAKE, FAKE, 100, None) == EWS
    assert f(FAKE_ODD, 0, 4, 8, FAKE, FAKE, FAKE, ws, None) == EALIGN     # fp32 at 2 bytes
    assert f(FAKE, 0, 4, 8, FAKE, FAKE, FAKE_ODD, ws, None) == EALIGN


def test_quantize_acts_validation(lib):
    f = lib.bitnet_quantize_acts
    assert f(FAKE, 5, 2, 8, FAKE, FAKE, None) == EDTYPE
    assert f(FAKE, 0, -1, 8, FAKE, FAKE, None) == ESHAPE
    assert f(None, 0, 0, 8, None, None, None) == OK          # M == 0: nothing to do
    assert f(None, 0, 2, 8, FAKE, FAKE, None) == ENULL
    assert f(FAKE, 0, 2, 8, FAKE, None, None) == ENULL
    assert f(FAKE_ODD, 0, 2, 8, FAKE, FAKE, None) == EALIGN


def test_ternary_linear_validation(lib):
    f = lib.bitnet_ternary_linear
    assert f(FAKE, FAKE, None, FAKE, 2, 3, 8, FAKE, 0, None, None) == ENULL
    assert f(FAKE, None, FAKE, FAKE, 2, 3, 8, FAKE, 0, None, None) == ENULL
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 8, None, 0, None, None) == ENULL
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 8, FAKE, 2, None, None) == EDTYPE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 6, FAKE, 0, None, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, -2, 3, 8, FAKE, 0, None, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 1 << 20, FAKE, 0, None, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 8, FAKE_ODD, 0, None, None) == EALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 3, 8, FAKE, 0, FAKE_ODD, None) == EALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 3, 8, FAKE, 0, None, None) == OK   # empty batch
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 0, 8, FAKE, 0, None, None) == OK   # no outputs
    assert f(None, None, FAKE, FAKE, 2, 0, 8, None, 0, None, None) == OK   # ... nothing to point at
    assert f(None, None, None, None, 0, 3, 8, None, 0, None, None) == OK


def test_quant_linear_validation(lib):
    f = lib.bitnet_quant_linear
    assert f(FAKE, FAKE, None, 0, 1, 3, 8, FAKE, FAKE, FAKE, 0, None, None) == ENULL
    assert f(FAKE, FAKE, FAKE, 0, 1, 3, 8, None, FAKE, FAKE, 0, None, None) == ENULL
    assert f(FAKE, FAKE, FAKE, 4, 1, 3, 8, FAKE, FAKE, FAKE, 0, None, None) == EDTYPE
    assert f(FAKE, FAKE, FAKE, 0, 1, 3, 10, FAKE, FAKE, FAKE, 0, None, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE_ODD, 0, 1, 3, 8, FAKE, FAKE, FAKE, 0, None, None) == EALIGN
    assert f(FAKE, FAKE, FAKE, 0, 0, 3, 8, FAKE, FAKE, FAKE, 0, None, None) == OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(N, "_lib", None)
    monkeypatch.setattr(N, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        N.lib()


def test_prologue_validation(lib):
    """The activation prologue's operands are checked before any HIP call."""
    P = N.BitnetActPrologue
    q = lib.bitnet_quantize_acts_ex
    assert q(FAKE, 0, ctypes.byref(P(None, 0x10000, 1e-5)), 2, 0, FAKE, FAKE, None) == ESHAPE  # norm needs K >= 1
    assert q(FAKE, 0, ctypes.byref(P(None, 0x10000, -1.0)), 2, 8, FAKE, FAKE, None) == ESHAPE
    assert q(FAKE, 0, ctypes.byref(P(None, 0x10000, float("nan"))), 2, 8, FAKE, FAKE, None) == ESHAPE
    assert q(FAKE, 0, ctypes.byref(P(None, 0x10002, 1e-5)), 2, 8, FAKE, FAKE, None) == EALIGN
    assert q(FAKE, 0, ctypes.byref(P(0x10002, None, 1e-5)), 2, 8, FAKE, FAKE, None) == EALIGN
    assert q(FAKE, 0, ctypes.byref(P(0x10002, None, 1e-5)), 0, 8, FAKE, FAKE, None) == OK  # M == 0
    mats = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10000, 0x10000, 3, 0x10000, None))
    f = lib.bitnet_quant_linear_ex
    assert f(mats, 1, FAKE, 0, ctypes.byref(P(None, 0x10002, 1e-5)), 1, 8, FAKE, FAKE, 0, None) == EALIGN
    assert f(mats, 1, FAKE, 0, ctypes.byref(P(None, 0x10000, float("inf"))), 1, 8, FAKE, FAKE, 0,
             None) == ESHAPE
    assert f(mats, 1, FAKE, 7, ctypes.byref(P(None, 0x10000, 1e-5)), 1, 8, FAKE, FAKE, 0, None) == EDTYPE


def test_t1_sizes_and_validation(lib):
    assert lib.bitnet_t1_packed_bytes(2560, 6912) == 2560 * 16 * 87
    assert lib.bitnet_t1_packed_bytes(3, 80) == 48
    assert lib.bitnet_t1_packed_bytes(3, 1) == 48
    assert lib.bitnet_t1_packed_bytes(-1, 80) == 0
    q = lib.bitnet_quantize_weights_t1
    ws = lib.bitnet_quantize_weights_workspace_bytes(4, 8)
    assert q(None, 0, 4, 8, FAKE, FAKE, FAKE, ws, None) == ENULL
    assert q(FAKE, 9, 4, 8, FAKE, FAKE, FAKE, ws, None) == EDTYPE
    assert q(FAKE, 0, 4, 0, FAKE, FAKE, FAKE, ws, None) == ESHAPE
    assert q(FAKE, 0, 4, 8, FAKE, FAKE, FAKE, 16, None) == EWS
    assert q(FAKE, 0, 4, 8, FAKE_ODD, FAKE, FAKE, ws, None) == EALIGN
    r = lib.bitnet_repack_t1
    assert r(None, 4, 8, FAKE, None) == ENULL
    assert r(FAKE, 4, 6, FAKE, None) == ESHAPE
    assert r(FAKE, -1, 8, FAKE, None) == ESHAPE
    assert r(FAKE, 4, 8, FAKE_ODD, None) == EALIGN
    assert r(FAKE, 0, 8, FAKE, None) == OK            # N == 0: nothing to do
    m = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10000, 0x10000, 8, 0x10000, 0))
    modd = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10002, 0x10000, 8, 0x10000, 0))
    t = lib.bitnet_ternary_linear_t1
    assert t(m, 1, FAKE, FAKE, 1, 100, 0, None) == ESHAPE    # K % 16 != 0
    assert t(m, 1, FAKE, FAKE, 1, 0, 0, None) == ESHAPE      # K < 16
    assert t(m, 1, FAKE, FAKE, 1, 131072 + 16, 0, None) == ESHAPE  # K > BITNET_MAX_K
    assert t(modd, 1, FAKE, FAKE, 1, 96, 0, None) == EALIGN  # weights not 16-byte aligned
    assert t(m, 1, FAKE_ODD, FAKE, 1, 96, 0, None) == EALIGN
    assert t(m, 1, None, FAKE, 1, 96, 0, None) == ENULL
    assert t(m, 1, FAKE, FAKE, 0, 96, 0, None) == OK         # M == 0: nothing to do
    f = lib.bitnet_quant_linear_t1
    assert f(m, 1, FAKE, 0, None, 1, 100, FAKE, FAKE, 0, None) == ESHAPE
    assert f(m, 1, FAKE, 7, None, 1, 96, FAKE, FAKE, 0, None) == EDTYPE
    assert f(modd, 1, FAKE, 0, None, 1, 96, FAKE, FAKE, 0, None) == EALIGN
    assert f(m, 1, FAKE, 0, None, 0, 96, FAKE, FAKE, 0, None) == OK


def test_lut_validation(lib):
    assert lib.bitnet_lut_workspace_bytes(2560, 6912) == 16 * 6912 + 2560 * 4
    assert lib.bitnet_lut_workspace_bytes(3, 64) == 1024 + 256
    assert lib.bitnet_lut_workspace_bytes(-1, 64) == 0
    f = lib.bitnet_ternary_linear_lut
    ws = lib.bitnet_lut_workspace_bytes(8, 64)
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 9, None, FAKE, ws, None) == EDTYPE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 96, FAKE, 0, None, FAKE, ws, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 8, 64, FAKE, 0, None, FAKE, ws, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 8, 64, FAKE, 0, None, FAKE, ws, None) == OK
    assert f(None, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 0, None, FAKE, ws, None) == ENULL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 0, None, None, ws, None) == EWS
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 0, None, FAKE, ws - 1, None) == EWS
    assert f(FAKE_ODD, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 0, None, FAKE, ws, None) == EALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 64, FAKE, 0, None, FAKE_ODD, ws, None) == EALIGN


# ---------------------------------------------------------------------------
# the Python binding validates every caller-supplied output before the C call
# ---------------------------------------------------------------------------

class _NoCall:
    """Stands in for the library: any call means validation let a bad tensor through."""
    def __getattr__(self, name):
        if name == "bitnet_t1_packed_bytes":
            return lambda n, k: n * 16 * ((k + 79) // 80)
        if name.endswith("_workspace_bytes"):
            return lambda n, k: 1 << 20
        def call(*a):
            raise AssertionError(f"{name} reached the C library with a bad tensor")
        return call


@pytest.fixture
def cpu_binding(monkeypatch):
    monkeypatch.setattr(N, "_need_cuda", lambda *ts: None)
    monkeypatch.setattr(N, "lib", lambda: _NoCall())
    return N


def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("case", [
    "y_dtype_mixed", "y_short", "acc_dtype", "acc_short", "xq_short", "xscale_short",
    "packed_short"])
def test_binding_rejects_bad_outputs_multi(cpu_binding, case):
    import torch
    m, k, n0, n1 = 2, 64, 32, 16
    x = _t((m, k), torch.float32)
    w0, w1 = _t((n0, k // 4), torch.uint8), _t((n1, k // 4), torch.uint8)
    s = _t((1,), torch.float32)
    y0, y1 = _t((m, n0), torch.float32), _t((m, n1), torch.float32)
    acc1 = _t((m, n1), torch.int32)
    x_q, x_scale = _t((m, k), torch.int8), _t((m,), torch.float32)
    if case == "y_dtype_mixed":
        y1 = _t((m, n1), torch.bfloat16)
    elif case == "y_short":
        y1 = _t((m, n1 - 1), torch.float32)
    elif case == "acc_dtype":
        acc1 = _t((m, n1), torch.float32)
    elif case == "acc_short":
        acc1 = _t((m - 1, n1), torch.int32)
    elif case == "xq_short":
        x_q = _t((m, k - 4), torch.int8)
    elif case == "xscale_short":
        x_scale = _t((m - 1,), torch.float32)
    elif case == "packed_short":
        w1 = _t((n1, k // 4 - 1), torch.uint8)
    with pytest.raises(ValueError):
        cpu_binding.bitnet_quant_linear_multi([(w0, s, y0), (w1, s, y1, acc1)], x, x_q=x_q,
                                              x_scale=x_scale)


def test_binding_rejects_bad_outputs_single(cpu_binding):
    import torch
    m, k, n = 3, 64, 8
    w, s = _t((n, k // 4), torch.uint8), _t((1,), torch.float32)
    xq, xs = _t((m, k), torch.int8), _t((m,), torch.float32)
    bad = [dict(y=_t((m, n + 1), torch.float32)), dict(y=_t((m, n), torch.float16)),
           dict(acc_out=_t((m, n), torch.int64)), dict(acc_out=_t((m, n - 1), torch.int32))]
    for kw in bad:
        with pytest.raises(ValueError):
            cpu_binding.bitnet_ternary_linear(w, s, xq, xs, **kw)
    with pytest.raises(ValueError):
        cpu_binding.bitnet_ternary_linear(w, s, xq, _t((m + 1,), torch.float32))
    with pytest.raises(ValueError):
        cpu_binding.bitnet_ternary_linear(w, _t((1,), torch.float64), xq, xs)
    x = _t((m, k), torch.float32)
    for kw in (dict(x_q=_t((m, k), torch.uint8)), dict(x_scale=_t((m,), torch.bfloat16)),
               dict(y=_t((n, m), torch.float32))):
        with pytest.raises(ValueError):
            cpu_binding.bitnet_quant_linear(w, s, x, **kw)
    with pytest.raises(ValueError):
        cpu_binding.bitnet_quantize_acts(x, x_q=_t((m, k - 1), torch.int8))
    with pytest.raises(ValueError):
        cpu_binding.bitnet_quantize_acts(x, norm_weight=_t((k + 1,), torch.float32))
    with pytest.raises(ValueError):
        cpu_binding.bitnet_quantize_weights(_t((n, k), torch.float32),
                                            packed=_t((n, k // 4 - 1), torch.uint8))
    with pytest.raises(ValueError):
        cpu_binding.bitnet_quantize_weights(_t((n, k), torch.float32),
                                            scale=_t((0,), torch.float32))


def test_binding_rejects_bad_outputs_t1_lut(cpu_binding):
    import torch
    m, k, n = 2, 160, 8
    rb = 16 * ((k + 79) // 80)
    s = _t((1,), torch.float32)
    xq, xs = _t((m, k), torch.int8), _t((m,), torch.float32)
    with pytest.raises(ValueError):   # a 2-bit matrix handed to the T1 call
        cpu_binding.bitnet_ternary_linear_t1([(_t((n, k // 4), torch.uint8), s)], xq, xs)
    with pytest.raises(ValueError):
        cpu_binding.bitnet_ternary_linear_t1([(_t((n, rb), torch.uint8), s,
                                               _t((m, n), torch.int32))], xq, xs)
    with pytest.raises(ValueError):
        cpu_binding.bitnet_repack_t1(_t((n, k // 4), torch.uint8), out=_t((n, rb - 16), torch.uint8))
    k = 128
    with pytest.raises(ValueError):
        cpu_binding.bitnet_ternary_linear_lut(_t((n, k // 4), torch.uint8), s,
                                              _t((m, k), torch.int8), _t((m,), torch.float32),
                                              y=_t((m, n), torch.int32), workspace=_t((1,), torch.uint8))


def test_chain_plan_validation(lib):
    """bitnet_chain_plan rejects bad stages before any HIP call (FAKE pointers are
    never dereferenced)."""
    plan_bytes = lib.bitnet_chain_plan_bytes(2)
    assert plan_bytes > 4096 and lib.bitnet_chain_plan_bytes(0) == 0
    mats = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10000, 0x10000, 64, 0x10000, None))

    def stage(**kw):
        f = dict(x=0x10000, x_dtype=0, y_dtype=0, K=256, mats=mats, count=1, x_q=0x10000,
                 x_scale=0x10000)
        f.update(kw)
        return N.BitnetChainStage(f["x"], f["x_dtype"], f["y_dtype"], f["K"], f["mats"],
                                  f["count"], f["x_q"], f["x_scale"])

    def plan(st, m=1, nbytes=plan_bytes, ptr=0x10000):
        arr = (N.BitnetChainStage * len(st))(*st)
        h = N.BitnetChain()
        return lib.bitnet_chain_plan(arr, len(st), m, ctypes.c_void_p(ptr), nbytes, ctypes.byref(h))

    assert lib.bitnet_chain_plan(None, 1, 1, FAKE, plan_bytes, None) == ENULL
    assert plan([stage()], m=0) == ESHAPE
    assert plan([stage()], m=5) == ESHAPE
    assert plan([stage(), stage()], nbytes=plan_bytes - 1) == EWS
    assert plan([stage()], ptr=0x10010) == EALIGN
    assert plan([stage(K=100)]) == ESHAPE
    assert plan([stage(K=65536)]) == ESHAPE
    assert plan([stage(count=0)]) == ESHAPE
    assert plan([stage(count=5)]) == ESHAPE
    assert plan([stage(x_dtype=7)]) == EDTYPE
    assert plan([stage(x=0x10008)]) == EALIGN
    assert plan([stage(x_q=0x10004)]) == EALIGN
    assert plan([stage(x=None)]) == ENULL
    bad = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10008, 0x10000, 64, 0x10000, None))
    assert plan([stage(mats=bad)]) == EALIGN
    zero_n = (N.BitnetMatrix * 1)(N.BitnetMatrix(0x10000, 0x10000, 0, 0x10000, None))
    assert plan([stage(mats=zero_n)]) == ESHAPE
    h = N.BitnetChain()
    assert lib.bitnet_chain_run(ctypes.byref(h), None) == ENULL
    h.plan = 0x10000
    h.n_stages, h.M, h.grid, h.kmax, h.tmax, h.ring = 1, 1, 1, 256, 1, 5
    assert lib.bitnet_chain_run(ctypes.byref(h), None) == ESHAPE
