"""The layer entry points of include/tlglayer.h: exported by the library, and every argument error caught on the
host before any launch (fake device addresses are never dereferenced).  No GPU needed."""

import ctypes
import os
import re

from dense_gemm_transformer_amd import layer, tlgemm as t

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tlglayer.h")


def test_library_exports_every_declared_layer_symbol():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tlg_\w+)\s*\(", text)))
    assert set(names) == set(layer.EXPORTS)
    lib = ctypes.CDLL(t.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def _ln(*a):
    return layer._lib.tlg_layernorm(*a)


def _att(*a):
    return layer._lib.tlg_attention(*a)


G = 1 << 32  # a fake, well-aligned device address


def test_layernorm_argument_errors():
    assert _ln(None, G, 2 * G, 3 * G, None, None, 4, 768, 1e-5, t.F32, None) == t.ERR_INVALID_ARG
    assert _ln(G, G + 8192, G + 16384, 3 * G, None, None, 0, 768, 1e-5, t.F32, None) == t.ERR_INVALID_ARG
    assert _ln(G, 2 * G, 3 * G, 4 * G, None, None, 4, 768, -1.0, t.F32, None) == t.ERR_INVALID_ARG
    assert _ln(G, 2 * G, 3 * G, 4 * G, None, None, 4, 768, 1e-5, 7, None) == t.ERR_INVALID_ARG
    assert _ln(G, 2 * G, 3 * G, 4 * G, None, None, 4, 4097, 1e-5, t.F32, None) == t.ERR_UNSUPPORTED
    assert _ln(G + 2, 2 * G, 3 * G, 4 * G, None, None, 4, 768, 1e-5, t.F32, None) == t.ERR_MISALIGNED
    assert _ln(G, 2 * G, 3 * G, 4 * G, G + 2, None, 4, 768, 1e-5, t.F32, None) == t.ERR_MISALIGNED
    assert _ln(G, 2 * G, 3 * G, G + 64, None, None, 4, 768, 1e-5, t.F32, None) == t.ERR_INVALID_ARG  # Y overlaps X
    assert _ln(G, 2 * G, 3 * G, 4 * G, 4 * G + 8, None, 4, 768, 1e-5, t.F32, None) == t.ERR_INVALID_ARG  # mean in Y
    assert _ln(G, 2 * G, 3 * G, 4 * G, 5 * G, 5 * G + 8, 4, 768, 1e-5, t.F32, None) == t.ERR_INVALID_ARG  # rstd in mean


def test_attention_argument_errors():
    ok = (64, 128, 12, 64)
    assert _att(None, 2 * G, None, *ok, t.F32, 1, None) == t.ERR_INVALID_ARG
    assert _att(G, 2 * G, None, 0, 128, 12, 64, t.F32, 1, None) == t.ERR_INVALID_ARG
    assert _att(G, 2 * G, None, 64, 128, 12, 32, t.F32, 1, None) == t.ERR_UNSUPPORTED  # head size
    assert _att(G, 2 * G, None, 64, 257, 12, 64, t.F32, 1, None) == t.ERR_UNSUPPORTED  # T
    assert _att(G + 4, 2 * G, None, *ok, t.F32, 1, None) == t.ERR_MISALIGNED
    assert _att(G, 2 * G + 8, None, *ok, t.F32, 1, None) == t.ERR_MISALIGNED
    assert _att(G, G + 1024, None, *ok, t.F32, 1, None) == t.ERR_INVALID_ARG  # out overlaps qkv
    assert _att(G, 2 * G, G + 4096, *ok, t.F32, 1, None) == t.ERR_INVALID_ARG  # lse overlaps qkv
    assert "head_size 64" in t.gemm_last_error() or "overlaps" in t.gemm_last_error()
