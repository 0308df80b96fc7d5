"""The C-ABI library without a GPU: it loads, exports every symbol that
include/bsgemm.h declares, and rejects malformed calls on the host before any
launch (these calls never reach the HIP runtime, so they run on any machine).

Every call below is either rejected by validation or has zero rows: none may
be a well-formed call with work in it, since the pointers are fake.
"""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_bsgemm_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsgemm.h")

INV, UNS, OK = bs.BS_ERR_INVALID, bs.BS_ERR_UNSUPPORTED, bs.BS_OK
P = 0x100000  # a fake, 16-byte aligned "device" address: never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bs.LIB_PATH):
        from block_scaled_fp8_bsgemm_amd import _build
        _build.build()
    return bs.load()


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:bs_status|const char \*)\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_exports():
    assert sorted(header_functions()) == sorted(bs.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in (OK, INV, UNS, bs.BS_ERR_LAUNCH):
        assert len(bs.status_str(st)) > 0
    assert bs.status_str(OK) == "ok"


def gemm(L, A=P, sa=P + 0x100000, B=P + 0x200000, sb=P + 0x300000, C=P + 0x1000000,
         M=256, N=512, K=256, bands=1, stride=0):
    return L.bsgemm_fp8(A, sa, B, sb, C, M, N, K, bands, stride, None)


def test_gemm_rejections(L):
    assert gemm(L, A=0) == INV and gemm(L, C=0) == INV and gemm(L, sb=0) == INV
    assert gemm(L, M=-1) == INV and gemm(L, N=0) == INV and gemm(L, K=0) == INV
    assert gemm(L, bands=0) == INV and gemm(L, stride=-8) == INV
    assert gemm(L, N=500) == UNS and gemm(L, K=200) == UNS
    assert gemm(L, bands=65) == UNS and gemm(L, M=250, bands=8) == UNS
    assert gemm(L, bands=2, stride=128 * 512 - 8) == UNS      # stride below band size
    assert gemm(L, bands=2, stride=128 * 512 + 4) == UNS      # stride not a multiple of 8
    assert gemm(L, A=P + 8) == UNS and gemm(L, C=P + 0x1000002) == UNS and gemm(L, sa=P + 0x100002) == UNS
    assert gemm(L, K=1 << 23) == UNS
    # output overlapping an input
    assert gemm(L, C=P + 1024) == INV
    assert gemm(L, C=P + 0x200000 + 4096) == INV
    # M = 0 is a no-op that touches nothing
    assert gemm(L, M=0) == OK


def test_reduce_rejections(L):
    parts = (ctypes.c_void_p * 4)(P, P + 0x100000, P + 0x200000, P + 0x300000)
    f = L.band_reduce
    assert f(None, 4, P + 0x1000000, 16, 64, None) == INV
    assert f(parts, 0, P + 0x1000000, 16, 64, None) == INV
    assert f(parts, 17, P + 0x1000000, 16, 64, None) == INV
    assert f(parts, 4, 0, 16, 64, None) == INV
    assert f(parts, 4, P + 0x1000000, -1, 64, None) == INV
    assert f(parts, 4, P + 0x1000000, 16, 60, None) == UNS
    assert f(parts, 4, P + 0x1000008, 16, 64, None) == UNS
    bad = (ctypes.c_void_p * 2)(P, 0)
    assert f(bad, 2, P + 0x1000000, 16, 64, None) == INV
    assert f(parts, 4, P + 0x100000 + 16, 16, 64, None) == INV   # out overlaps part 1
    assert f(parts, 4, P + 0x1000000, 0, 64, None) == OK


def test_rowq_rowdq_blockq_rejections(L):
    assert L.rowq_e4m3(0, P + 0x100000, P + 0x200000, 4, 64, None) == INV
    assert L.rowq_e4m3(P, P + 0x100000, P + 0x200000, 4, 60, None) == UNS
    assert L.rowq_e4m3(P, P + 0x100004, P + 0x200000, 4, 64, None) == UNS
    assert L.rowq_e4m3(P, P + 64, P + 0x200000, 4, 64, None) == INV         # q overlaps x
    assert L.rowq_e4m3(P, P + 0x100000, P + 0x100000 + 32, 4, 64, None) == INV  # scale overlaps q
    assert L.rowq_e4m3(P, P + 0x100000, P + 0x200000, 0, 64, None) == OK
    assert L.rowdq_e4m3(P, P + 0x100000, 0, 4, 64, None) == INV
    assert L.rowdq_e4m3(P, P + 0x100000, P + 0x200000, 4, -64, None) == INV
    assert L.rowdq_e4m3(P, P + 0x100002, P + 0x200000, 4, 64, None) == UNS
    assert L.rowdq_e4m3(P, P + 0x100000, P + 128, 4, 64, None) == INV        # y overlaps q
    assert L.rowdq_e4m3(P, P + 0x100000, P + 0x200000, 0, 64, None) == OK
    assert L.blockq_e4m3(P, P + 0x100000, P + 0x200000, 4, 256, 2, None) == UNS
    assert L.blockq_e4m3(P, P + 0x100000, P + 0x200000, 4, 200, 1, None) == UNS
    assert L.blockq_e4m3(P, P + 0x100000, 0, 4, 256, 1, None) == INV
    assert L.blockq_e4m3(P, P + 512, P + 0x200000, 4, 256, 1, None) == INV
    assert L.blockq_e4m3(P, P + 0x100000, P + 0x200000, 0, 256, 128, None) == OK


def test_actq_rejections(L):
    f = L.actq_e4m3
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p]
    assert f(0, P + 0x100000, P + 0x200000, 4, 256, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, -1, 256, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, 4, 0, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, 4, 200, None) == UNS             # cols % 128
    assert f(P + 8, P + 0x100000, P + 0x200000, 4, 256, None) == UNS         # x alignment
    assert f(P, P + 0x100000, P + 0x200002, 4, 256, None) == UNS             # scale alignment
    assert f(P, P + 1024, P + 0x200000, 4, 256, None) == INV                 # q overlaps x (2 KiB)
    assert f(P, P + 0x100000, P + 0x100000 + 512, 4, 256, None) == INV       # scale overlaps q
    assert f(P, P + 0x100000, P + 0x200000, 0, 256, None) == OK


def mxgemm(L, A=P, sa=P + 0x100000, B=P + 0x200000, sb=P + 0x300000, C=P + 0x1000000,
           M=256, N=512, K=256, bands=1, stride=0):
    return L.mxgemm_fp8(A, sa, B, sb, C, M, N, K, bands, stride, None)


def test_mxgemm_rejections(L):
    assert mxgemm(L, A=0) == INV and mxgemm(L, sa=0) == INV and mxgemm(L, sb=0) == INV
    assert mxgemm(L, C=0) == INV and mxgemm(L, M=-1) == INV and mxgemm(L, N=0) == INV
    assert mxgemm(L, K=0) == INV and mxgemm(L, bands=0) == INV and mxgemm(L, stride=-8) == INV
    assert mxgemm(L, N=500) == UNS and mxgemm(L, K=160) == UNS            # K % 128
    assert mxgemm(L, bands=65) == UNS and mxgemm(L, M=250, bands=8) == UNS
    assert mxgemm(L, bands=2, stride=128 * 512 - 8) == UNS
    assert mxgemm(L, A=P + 8) == UNS and mxgemm(L, C=P + 0x1000002) == UNS
    assert mxgemm(L, sa=P + 0x100002) == UNS and mxgemm(L, sb=P + 0x300001) == UNS
    assert mxgemm(L, K=1 << 23) == UNS
    assert mxgemm(L, C=P + 1024) == INV                                     # C over A
    assert mxgemm(L, C=P + 0x300000 + 64) == INV                           # C over b_scale
    assert mxgemm(L, M=0) == OK


def test_mxq_rejections(L):
    f = L.mxq_e4m3
    assert f(0, P + 0x100000, P + 0x200000, 4, 256, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, -1, 256, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, 4, 0, None) == INV
    assert f(P, P + 0x100000, P + 0x200000, 4, 48, None) == UNS              # cols % 32
    assert f(P + 8, P + 0x100000, P + 0x200000, 4, 256, None) == UNS         # x alignment
    assert f(P, P + 0x100008, P + 0x200000, 4, 256, None) == UNS             # q alignment
    assert f(P, P + 1024, P + 0x200000, 4, 256, None) == INV                 # q overlaps x (2 KiB)
    assert f(P, P + 0x100000, P + 0x100000 + 512, 4, 256, None) == INV       # scale overlaps q
    assert f(P, P + 0x100000, P + 0x200001, 0, 256, None) == OK              # scales: byte aligned


def test_gemm_pb_rejections(L):
    def g(**kw):
        a = dict(A=P, sa=P + 0x100000, B=P + 0x200000, sb=P + 0x300000, C=P + 0x1000000,
                 M=256, N=512, K=256, bands=1, stride=0)
        a.update(kw)
        return L.bsgemm_fp8_pb(a["A"], a["sa"], a["B"], a["sb"], a["C"], a["M"], a["N"], a["K"],
                               a["bands"], a["stride"], None)
    assert g(B=0) == INV and g(M=-1) == INV and g(bands=0) == INV
    assert g(N=500) == UNS and g(K=200) == UNS and g(M=250, bands=8) == UNS
    assert g(B=P + 0x200008) == UNS and g(sb=P + 0x300002) == UNS
    assert g(C=P + 0x200000 + 4096) == INV                  # C over the prepacked weight
    assert g(M=0) == OK


def test_bprepack_rejections(L):
    f = L.bprepack_e4m3
    assert f(0, P + 0x100000, 512, 256, None) == INV
    assert f(P, 0, 512, 256, None) == INV
    assert f(P, P + 0x100000, 0, 256, None) == INV and f(P, P + 0x100000, 512, -128, None) == INV
    assert f(P, P + 0x100000, 500, 256, None) == UNS                      # N % 128
    assert f(P, P + 0x100000, 512, 200, None) == UNS                      # K % 128
    assert f(P, P + 0x100000, 512, 1 << 23, None) == UNS
    assert f(P + 8, P + 0x100000, 512, 256, None) == UNS                  # alignment
    assert f(P, P + 0x100008, 512, 256, None) == UNS
    assert f(P, P, 512, 256, None) == INV                                 # in place
    assert f(P, P + 512 * 256 - 16, 512, 256, None) == INV               # overlapping


def test_band_rowq_rejections(L):
    parts = (ctypes.c_void_p * 4)(P, P + 0x100000, P + 0x200000, P + 0x300000)
    f = L.band_rowq_e4m3
    Q, S = P + 0x1000000, P + 0x2000000
    assert f(None, 4, Q, S, 64, 1024, None) == INV
    assert f(parts, 0, Q, S, 64, 1024, None) == INV and f(parts, 17, Q, S, 64, 1024, None) == INV
    assert f(parts, 4, 0, S, 64, 1024, None) == INV and f(parts, 4, Q, 0, 64, 1024, None) == INV
    assert f(parts, 4, Q, S, -1, 1024, None) == INV and f(parts, 4, Q, S, 64, 0, None) == INV
    assert f(parts, 4, Q, S, 64, 1020, None) == UNS                 # N % 8
    assert f(parts, 4, Q, S, 64, 8200, None) == UNS                 # N > 8192
    assert f(parts, 4, Q, S, 1 << 31, 8, None) == UNS               # one workgroup per row: rows < 2^31
    assert f(parts, 4, Q + 8, S, 64, 1024, None) == UNS and f(parts, 4, Q, S + 2, 64, 1024, None) == UNS
    assert f(parts, 4, P + 4096, S, 64, 1024, None) == INV          # q over part 0
    assert f(parts, 4, Q, Q + 1024, 64, 1024, None) == INV          # scale over q
    assert f(parts, 4, Q, S, 0, 1024, None) == OK
