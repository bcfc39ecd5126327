"""The C-ABI library loads and exports every function include/lsa.h declares
(CPU only: no compute call is made)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")
LIB = os.path.join(ROOT, "learned_sparse_kv_amd", "liblsa.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_\w+)\s*\(", text)))


def test_header_declares_the_six_entry_points():
    names = declared()
    for n in ["lsa_score_chunks", "lsa_select_threshold", "lsa_topk_refine", "lsa_gather_kv",
              "lsa_sparse_decode_attn", "lsa_step64"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        from learned_sparse_kv_amd import build
        build.build()
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    from learned_sparse_kv_amd import lsa
    for code in (0, -1, -2, -3, -4, -5):
        assert lsa.lib().lsa_status_str(code).decode() == lsa._STATUS[code]
