"""The C ABI without a GPU: the library loads, exports every entry point
that include/qgemv.h declares, and refuses bad arguments by name before it
touches any pointer (0xdeadbeef pointers are never dereferenced)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = 0xDEADBEEF0  # 16-byte aligned, never mapped


@pytest.fixture(scope="module")
def q():
    import quantized_weight_decode_amd as q
    try:
        q.lib()
    except ImportError as e:
        pytest.skip(str(e))
    return q


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_\w+)\s*\(", src)))


def test_header_and_binding_agree(q):
    assert sorted(q.ENTRY_POINTS) == declared_entry_points()


def test_library_exports_every_declared_symbol(q):
    assert sorted(q.exported_symbols()) == declared_entry_points()


def test_strerror_names_every_status(q):
    for st in range(0, 9):
        assert q.strerror(st) and q.strerror(st) != "unknown status"
    assert q.strerror(99) == "unknown status"


def test_i4g_refusals(q):
    f = q.qgemv_i4g
    assert f(0, BAD, BAD, BAD, 1, 64, 8, 64, 0) == 1            # NULL
    assert f(BAD, BAD, BAD, BAD, 0, 64, 8, 64, 0) == 2          # S = 0
    assert f(BAD, BAD, BAD, BAD, 9, 64, 8, 64, 0) == 2          # S > 8
    assert f(BAD, BAD, BAD, BAD, 1, 0, 8, 64, 0) == 2           # I = 0
    assert f(BAD, BAD, BAD, BAD, 1, 64, -1, 64, 0) == 2         # O < 0
    assert f(BAD, BAD, BAD, BAD, 1, 64, 8, 63, 0) == 3          # odd gs
    assert f(BAD, BAD, BAD, BAD, 1, 64, 8, 0, 0) == 3           # gs = 0
    assert f(BAD, BAD + 2, BAD, BAD, 1, 64, 8, 64, 0) == 4      # misaligned scales
    assert f(BAD, BAD, BAD, BAD + 1, 1, 64, 8, 64, 0) == 4      # misaligned y
    assert q.qgemv_dequant_i4g(BAD, BAD, 0, 64, 8, 64, 0) == 1
    assert q.qgemv_dequant_i4g(BAD, BAD, BAD, 64, 8, 5, 0) == 3


def test_mq4_refusals(q):
    assert q.qgemv_mq4v2(BAD, BAD, BAD, 1, 300, 8, 0) == 5                 # I % 256
    assert q.qgemv_mq4v2(BAD, BAD, 0, 1, 256, 8, 0) == 1
    assert q.qgemv_fwht256(BAD, BAD, BAD + 4, 1, 256, 0) == 4              # x_rot misaligned
    r = q.qgemv_mq4v2_rot
    assert r(BAD, BAD, 0, BAD, 1, 256, 8, 0) == 1                          # NULL signs
    assert r(BAD, BAD, BAD, BAD, 9, 256, 8, 0) == 2                        # S > 8
    assert r(BAD, BAD, BAD, BAD, 1, 300, 8, 0) == 5                        # I % 256
    assert r(BAD, BAD, BAD + 4, BAD, 1, 256, 8, 0) == 4                    # signs misaligned
    assert r(BAD, BAD + 8, BAD, BAD, 1, 256, 8, 0) == 4                    # x misaligned
    assert r(BAD + 4, BAD, BAD, BAD, 1, 256, 8, 0) == 4                    # w misaligned
    assert r(BAD, BAD, BAD, BAD, 1, 65536, 8, 0) == 2                      # staging > LDS


def test_fp8_refusals(q):
    f = q.qgemv_fp8b128
    assert f(0, BAD, BAD, BAD, 1, 64, 8, 0) == 1
    assert f(BAD, BAD, BAD, BAD, 1, 64, 0, 0) == 2
    assert f(BAD, BAD + 1, BAD, BAD, 1, 64, 8, 0) == 4


def test_fp8_ue8m0_refusals(q):
    f = q.qgemv_fp8b128_ue8m0
    assert f(BAD, 0, BAD, BAD, 1, 64, 8, 0) == 1
    assert f(BAD, BAD, BAD, BAD, 0, 64, 8, 0) == 2
    assert f(BAD, BAD + 1, BAD + 2, BAD, 1, 64, 8, 0) == 4                 # x misaligned
    assert q.qgemv_dequant_fp8b128_ue8m0(BAD, BAD, BAD + 2, 64, 8, 0) == 4


def test_mq4_family_refusals(q):
    assert q.qgemv_mq4v1(BAD, BAD, BAD, 1, 300, 8, 0) == 5
    assert q.qgemv_mq4c(0, BAD, BAD, 1, 256, 8, 0) == 1
    assert q.qgemv_mq4c(BAD, BAD + 2, BAD, 1, 256, 8, 0) == 4
    assert q.qgemv_dequant_mq4v1(BAD, BAD, 300, 8, 0) == 5
    assert q.qgemv_dequant_mq4c(BAD, BAD + 1, 256, 8, 0) == 4
    e = q.qgemv_mq4v2_encode
    assert e(0, BAD, 256, 8, 0) == 1
    assert e(BAD, BAD, 300, 8, 0) == 5
    assert e(BAD + 4, BAD, 256, 8, 0) == 4                                   # W not 16-B aligned
    assert e(BAD, BAD + 4, 256, 8, 0) == 4                                   # out not 8-B aligned
    assert e(BAD, BAD, 256, 0, 0) == 2


def test_router_refusals(q):
    f = q.qgemv_router_topk
    assert f(0, 4, 256, 256, 8, BAD, BAD, 0) == 1
    assert f(BAD, 4, 2048, 2048, 8, BAD, BAD, 0) == 2                         # E > 1024
    assert f(BAD, 4, 256, 200, 8, BAD, BAD, 0) == 2                           # ld < E
    assert f(BAD, 4, 256, 256, 65, BAD, BAD, 0) == 2                          # K > 64
    assert f(BAD, 4, 4, 4, 5, BAD, BAD, 0) == 2                               # K > E
    assert f(BAD + 2, 4, 256, 256, 8, BAD, BAD, 0) == 4


def test_prefill_refusals(q):
    f = q.qgemv_i4g_prefill
    assert f(0, BAD, BAD, BAD, 64, 512, 8, 64, 0) == 1
    assert f(BAD, BAD, BAD, BAD, 0, 512, 8, 64, 0) == 2
    assert f(BAD, BAD, BAD, BAD, 64, 512, 8, 63, 0) == 3
    assert f(BAD, BAD + 2, BAD, BAD, 64, 512, 8, 64, 0) == 4
