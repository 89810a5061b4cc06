"""The C-ABI library loads, exports every symbol include/cb.h declares, and
rejects bad arguments with the documented status before touching a device."""
import ctypes as C
import os
import re

import pytest

from chunked_prefill_attention_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cb.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported_and_bound():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding declarations differ from the header"


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.cb_status_string(0) == b"CB_OK"
    assert lib.cb_status_string(-3) == b"CB_ERR_WORKSPACE"
    assert lib.cb_abi_version() == 4


NULL = C.c_void_p(0)
FAKE = C.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _step(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, stride=64, qsl=FAKE, ctx=FAKE, off=FAKE, B=2, nd=1, T=5,
             maxctx=1000, hq=8, hkv=2, d=128, page=16, pages=100, scale=0.088, window=0, dtype=1, out=FAKE,
             ws=FAKE, wsb=0, stream=NULL)
    a.update(over)
    lib = _lib.load()
    return lib.cb_attention_step(a["q"], a["k"], a["v"], a["bt"], a["stride"], a["qsl"], a["ctx"], a["off"],
                                 a["B"], a["nd"], a["T"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["page"],
                                 a["pages"], a["scale"], a["window"], a["dtype"], a["out"], a["ws"], a["wsb"],
                                 a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(page=32), -2), (dict(d=96), -2), (dict(dtype=2), -2), (dict(hq=7), -1), (dict(hq=64, hkv=2), -2),
    (dict(hkv=0), -1), (dict(nd=3), -1), (dict(T=0, nd=1), -1), (dict(q=NULL), -1), (dict(out=NULL), -1),
    (dict(bt=NULL), -1), (dict(stride=10), -1), (dict(pages=0), -1), (dict(scale=float("nan")), -1),
    (dict(maxctx=0), -1), (dict(wsb=16), -3), (dict(ws=NULL, wsb=1 << 30), -3), (dict(B=0, T=3, nd=0), -1),
    (dict(window=-1), -1),
])
def test_attention_step_rejects_bad_arguments(over, status):
    assert _step(**over) == status
    assert _lib.load().cb_last_error() != b""


def test_empty_step_is_a_noop():
    assert _step(T=0, nd=0, B=0) == 0


def test_workspace_bytes():
    lib = _lib.load()
    assert lib.cb_attention_workspace_bytes(2, 1, 5, 8, 2, 128, 1000, 0) == 0          # fp32: none
    n = lib.cb_attention_workspace_bytes(67, 64, 2048, 32, 8, 128, 8192, 1)
    assert 0 < n < (1 << 30)
    assert n >= lib.cb_attention_workspace_bytes(67, 64, 2048, 32, 8, 128, 4096, 1)
    assert lib.cb_attention_workspace_bytes(2, 3, 5, 8, 2, 128, 1000, 1) == C.c_size_t(-1).value
    assert lib.cb_attention_workspace_bytes(2, 1, 5, 7, 2, 128, 1000, 1) == C.c_size_t(-1).value


def test_kv_append_rejects_bad_arguments():
    lib = _lib.load()
    f = lib.cb_kv_append
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 128, 100, 8, 1, NULL) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 100, 100, 16, 1, NULL) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 100, 16, 1, NULL) == -1
    assert f(NULL, FAKE, FAKE, FAKE, FAKE, 10, 8, 128, 100, 16, 1, NULL) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 128, 0, 16, 1, NULL) == -1
    assert f(NULL, NULL, NULL, NULL, NULL, 0, 8, 128, 100, 16, 1, NULL) == 0   # empty: no-op


@pytest.mark.parametrize("scale", [0.0, -0.088, -0.0])
def test_bf16_rejects_non_positive_scale(scale):
    """The bf16 online softmax orders scores by their raw value, which matches
    the scaled order only for scale > 0: other scales are refused up front."""
    assert _step(scale=scale) == -2
    assert b"scale > 0" in _lib.load().cb_last_error()
