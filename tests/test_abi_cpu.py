"""Host-only checks of the C ABI: the library loads and exports every entry
point include/lce.h declares; workspace sizing and host-side argument checks
(which return before any HIP call).  No compute call runs here."""

import ctypes
import os
import re

import pytest

from lm_head_projection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_projection_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        getattr(raw, n)  # raises AttributeError if not exported


def test_status_strings(lib):
    for st in (0, 1, -1, -2, -3, -4, -5):
        assert lib.lce_status_string(st)
    assert b"C == 0" in lib.lce_status_string(1)


def test_workspace_size_never_scales_with_N_times_V(lib):
    BF16, F32 = _lib.LCE_DTYPE_BF16, _lib.LCE_DTYPE_F32
    assert lib.lce_workspace_size(-1, 8, 8, BF16) == 0
    assert lib.lce_workspace_size(8, 0, 8, BF16) == 0
    assert lib.lce_workspace_size(8, 8, 0, BF16) == 0
    assert lib.lce_workspace_size(8, 8, 8, 7) == 0
    for N, D, V in ((16384, 1024, 248320), (32768, 4096, 248320), (2048, 1024, 151936)):
        ws = lib.lce_workspace_size(N, D, V, BF16)
        nxv = N * V * 2
        assert 0 < ws < nxv / 2, (N, D, V, ws, nxv)
    # growing V does not grow the chunked store beyond its fixed width
    a = lib.lce_workspace_size(4096, 1024, 200_000, BF16)
    b = lib.lce_workspace_size(4096, 1024, 400_000, BF16)
    assert b - a < 4096 * 200_000  # only the per-row-block db partials grow with V
    assert lib.lce_workspace_size(64, 128, 1000, F32) > 0


def test_host_argument_checks_return_before_any_hip_call(lib):
    C = ctypes.c_int64(5)
    # null C_host / negative N / bad V
    assert lib.lce_compact_valid(None, None, 10, 100, -100, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    assert lib.lce_compact_valid(None, None, -1, 100, -100, None, ctypes.byref(C), None, 0, None) == _lib.LCE_ERR_ARG
    assert lib.lce_compact_valid(None, None, 10, 0, -100, None, ctypes.byref(C), None, 0, None) == _lib.LCE_ERR_ARG
    # N = 0 is an empty problem: C = 0
    assert lib.lce_compact_valid(None, None, 0, 10, -100, None, ctypes.byref(C), None, 0, None) == _lib.LCE_OK_EMPTY
    assert C.value == 0
    # forward: C > N, missing outputs, bad dtype
    args = [None] * 5
    assert lib.lce_forward(*args, 3, 2, 8, 8, 1, None, None, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    assert lib.lce_forward(*args, 1, 2, 8, 8, 9, None, None, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    # backward: dW missing
    assert lib.lce_backward(*args, 1, 2, 8, 8, 1, None, None, None, None, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    # reductions: unknown code, weights or a divisor outside SUM, negative / NaN / inf divisor
    w = (ctypes.c_float * 4)()
    out = (ctypes.c_float * 4)()
    fe, be = lib.lce_forward_ex, lib.lce_backward_ex
    assert fe(*args, 1, 2, 8, 8, 1, 7, None, 0.0, out, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    assert fe(*args, 1, 2, 8, 8, 1, _lib.LCE_REDUCTION_MEAN, w, 0.0, out, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    assert fe(*args, 1, 2, 8, 8, 1, _lib.LCE_REDUCTION_NONE, None, 3.0, out, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    for bad in (-1.0, float("nan"), float("inf")):
        assert fe(*args, 1, 2, 8, 8, 1, _lib.LCE_REDUCTION_SUM, w, bad, out, None, None, None, 0, None) == _lib.LCE_ERR_ARG
        assert be(*args, 1, 2, 8, 8, 1, _lib.LCE_REDUCTION_SUM, w, bad, None, None, None, None, None, None,
                  None, 0, None) == _lib.LCE_ERR_ARG
    assert be(*args, 1, 2, 8, 8, 1, 3, None, 0.0, None, None, None, None, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    # a valid reduction still rejects a missing loss output before any HIP call
    assert fe(*args, 1, 2, 8, 8, 1, _lib.LCE_REDUCTION_SUM, None, 0.0, None, None, None, None, 0, None) == _lib.LCE_ERR_ARG
    # vocabulary shards: P out of range, bounds not starting at 0 or not increasing, negative v_begin
    i64 = ctypes.c_int64
    loss1 = (ctypes.c_float * 1)()
    ws4 = (ctypes.c_float * 64)()
    good = (i64 * 3)(0, 5, 9)
    for P, bnd in ((0, good), (65, good), (2, (i64 * 3)(1, 5, 9)), (2, (i64 * 3)(0, 5, 5)), (2, (i64 * 3)(0, 7, 3))):
        assert lib.lce_merge_shards(out, P, bnd, None, None, 3, 4, _lib.LCE_REDUCTION_MEAN, None, 0.0, loss1,
                                    None, None, ws4, 256, None) == _lib.LCE_ERR_ARG
    assert lib.lce_merge_shards(out, 2, good, None, None, 3, 4, 9, None, 0.0, loss1, None, None, ws4, 256,
                                None) == _lib.LCE_ERR_ARG
    assert lib.lce_forward_shard(*args, 1, 2, 8, 8, -1, 1, out, None, 0, None) == _lib.LCE_ERR_ARG
    assert lib.lce_forward_shard(*args, 1, 2, 8, 8, 0, 1, None, None, 0, None) == _lib.LCE_ERR_ARG
    assert lib.lce_backward_shard(*args, 1, 2, 8, 8, -1, 1, 0, None, 0.0, None, None, None, None, None, None,
                                  None, 0, None) == _lib.LCE_ERR_ARG
    # gradient filter: eps negative / NaN / inf, unknown reduction -> ERR_ARG; fp32 -> UNSUPPORTED
    bf = lib.lce_backward_filtered
    for bad in (-1.0, float("nan"), float("inf")):
        assert bf(*args, 1, 2, 8, 8, 1, 0, None, 0.0, None, None, None, bad, 3, None, None, None, None, 0,
                  None) == _lib.LCE_ERR_ARG
    assert bf(*args, 1, 2, 8, 8, 1, 5, None, 0.0, None, None, None, 0.1, 3, None, None, None, None, 0,
              None) == _lib.LCE_ERR_ARG
    for which in (0, 2, 4, -1):
        assert bf(*args, 1, 2, 8, 8, 1, 0, None, 0.0, None, None, None, 0.1, which, None, None, None, None, 0,
                  None) == _lib.LCE_ERR_ARG
    assert bf(*args, 1, 2, 8, 8, _lib.LCE_DTYPE_F32, 0, None, 0.0, None, None, None, 0.1, 3, None, None, None,
              None, 0, None) == _lib.LCE_ERR_UNSUPPORTED
    # profiling switch validates its argument
    assert lib.lce_profile_start(0) == _lib.LCE_ERR_ARG
    assert lib.lce_profile_count() >= 0


def test_python_binding_names_match_c_abi():
    for n in ("lce_workspace_size", "lce_compact_valid", "lce_forward", "lce_backward", "lce_forward_ex",
              "lce_backward_ex", "lce_backward_filtered", "lce_forward_shard", "lce_merge_shards",
              "lce_backward_shard"):
        assert callable(getattr(_lib, n))


def test_wrapper_rejects_unknown_options_before_any_library_call():
    """The autograd wrapper refuses an unknown filter choice or reduction
    before it allocates or calls into the library (CPU tensors suffice)."""
    import torch
    from lm_head_projection_amd import linear_cross_entropy
    H = torch.zeros(4, 8)
    W = torch.zeros(5, 8)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        linear_cross_entropy(H, W, y, filter_eps=0.1, filter_grads="dw")
    with pytest.raises(KeyError):
        linear_cross_entropy(H, W, y, reduction="median")
