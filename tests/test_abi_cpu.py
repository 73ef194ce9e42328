"""The C ABI library on the CPU: it loads, exports every entry point include/pi.h declares,
and its host-only calls behave (no GPU work is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from activation_sparse_ffn_layer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib._SIGS), "binding and header disagree"


COMPUTE_CALLS = ("pi_predict", "pi_sparse_ffn", "pi_layer", "pi_compact", "pi_glue", "pi_stack_run",
                 "pi_stack_run_dump", "pi_stack_profile", "pi_hot_first_order", "pi_permute_rows", "pi_q4_dequant")


def test_every_compute_call_cites_the_pages():
    """The comment right above each compute call's declaration names the passage of the pages
    that defines the operation (P1/P2/P3 with a section in «», or a page's introduction or
    header bullets)."""
    text = open(HEADER).read()
    cite = re.compile(r"P[123] (?:«[^»]+»|intro|header)")
    for name in COMPUTE_CALLS:
        m = re.search(r"(/\*(?:(?!\*/).)*\*/)\s*pi_status\s+" + name + r"\s*\(", text, flags=re.S)
        assert m, f"{name}: no comment directly above its declaration"
        assert cite.search(m.group(1)), f"{name}: its comment cites no passage of the pages"


def test_abi_version_and_status_strings():
    L = _lib.lib()
    assert L.pi_abi_version() == 2
    assert L.pi_status_str(0) == b"ok"
    assert L.pi_status_str(1) == b"invalid argument"
    assert L.pi_last_error(None) == b""


def test_null_arguments_rejected_on_host():
    L = _lib.lib()
    assert L.pi_ctx_create(0, None, 1, 64, 64, 0, None) == _lib.PI_ERR_INVALID
    h = ctypes.c_void_p()
    assert L.pi_ctx_create(0, None, 0, 64, 64, 0, ctypes.byref(h)) == _lib.PI_ERR_INVALID
    assert L.pi_ctx_create(0, None, 1, 60, 64, 0, ctypes.byref(h)) == _lib.PI_ERR_INVALID
    assert L.pi_predict(None, None, None, 1, None, None, None, None) == _lib.PI_ERR_INVALID
    assert L.pi_hot_first_order(None, 4, None) == _lib.PI_ERR_INVALID
    assert L.pi_ctx_set_mask_mode(None, 1) == _lib.PI_ERR_INVALID
    assert L.pi_layer_noalloc(0, None, None, None, 1, None, None, None, None) == _lib.PI_ERR_INVALID


@pytest.mark.parametrize("ffn", [5, 64, 4096])
def test_hot_first_order_matches_oracle(ffn):
    from activation_sparse_ffn_layer_amd import hot_first_order
    rng = np.random.default_rng(ffn)
    p = rng.choice([0.01, 0.1, 0.5, 0.95], size=ffn) if ffn > 5 else np.array([0.1, 0.5, 0.1, 0.9, 0.5])
    np.testing.assert_array_equal(hot_first_order(p), oracle.hot_first_order(p))
