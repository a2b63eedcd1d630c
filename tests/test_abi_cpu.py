"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the GPU (every
call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

import bit_group_quantized_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:q4_status|int64_t|int|const char\*)\s+(q4_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = header_functions()
    assert names == sorted(q4.exported_symbols())
    for want in ("q4_pack", "q4_unpack", "q4_gemv", "q4_gemm_small", "q4_multilinear_step"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q4.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_layout_version_and_status_strings():
    assert q4.q4_layout_version() == 1
    assert q4.q4_status_str(0) == "ok"
    assert q4.q4_status_str(q4.Q4_ERR_ALIGN) == "misaligned pointer"
    assert q4.q4_status_str(99) == "unknown status"


A16 = 0x10000   # a 16-byte aligned fake address: validation fails before any use
ODD = 0x10001
Y16 = 0x400000  # another one, far from A16 (chain outputs must not overlap their own input)


def _p(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("case,want", [
    (dict(x=0), q4.Q4_ERR_NULL),
    (dict(packed=0), q4.Q4_ERR_NULL),
    (dict(scales=0), q4.Q4_ERR_NULL),
    (dict(biases=0), q4.Q4_ERR_NULL),
    (dict(y=0), q4.Q4_ERR_NULL),
    (dict(k=0), q4.Q4_ERR_SHAPE),
    (dict(k=48), q4.Q4_ERR_SHAPE),
    (dict(n=-1), q4.Q4_ERR_SHAPE),
    (dict(dtype=7), q4.Q4_ERR_SHAPE),
    (dict(x=ODD), q4.Q4_ERR_ALIGN),
    (dict(packed=A16 + 4), q4.Q4_ERR_ALIGN),
    (dict(scales=ODD), q4.Q4_ERR_ALIGN),
    (dict(y=ODD), q4.Q4_ERR_ALIGN),
    (dict(k=32 * 1024), q4.Q4_ERR_UNSUPPORTED),
    (dict(k=q4.MAX_K + 32), q4.Q4_ERR_UNSUPPORTED),  # one group past the widest supported row
])
def test_gemv_validation(case, want):
    a = dict(x=A16, packed=A16, scales=A16, biases=A16, n=16, k=64, y=A16, dtype=0)
    a.update(case)
    st = q4.load().q4_gemv(_p(a["x"]), _p(a["packed"]), _p(a["scales"]), _p(a["biases"]), a["n"], a["k"],
                           _p(a["y"]), a["dtype"], None)
    assert st == want


@pytest.mark.parametrize("m,want", [(0, q4.Q4_ERR_SHAPE), (17, q4.Q4_ERR_SHAPE), (-3, q4.Q4_ERR_SHAPE)])
def test_gemm_small_rejects_m(m, want):
    st = q4.load().q4_gemm_small(_p(A16), m, _p(A16), _p(A16), _p(A16), 16, 64, _p(A16), 0, None)
    assert st == want


@pytest.mark.parametrize("steps,step,want", [
    (16, 16, q4.Q4_ERR_SHAPE), (16, -1, q4.Q4_ERR_SHAPE), (0, 0, q4.Q4_ERR_SHAPE)])
def test_multilinear_rejects_step(steps, step, want):
    st = q4.load().q4_multilinear_step(_p(A16), 1, _p(A16), _p(A16), _p(A16), steps, 8, 64, step, _p(A16), 0,
                                       None)
    assert st == want


def test_pack_and_unpack_validation():
    lib = q4.load()
    assert lib.q4_pack(None, 4, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_pack(_p(ODD), 4, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_pack(_p(A16), 4, 40, _p(A16), _p(A16), _p(A16), None) == q4.Q4_ERR_SHAPE
    assert lib.q4_unpack(_p(A16), _p(A16), _p(A16), 4, 64, None, None, None) == q4.Q4_ERR_NULL
    assert lib.q4_unpack(_p(A16), _p(A16), _p(A16), 4, 64, _p(ODD), None, None) == q4.Q4_ERR_ALIGN


def test_empty_calls_are_noops():
    lib = q4.load()
    assert lib.q4_gemv(_p(A16), _p(A16), _p(A16), _p(A16), 0, 64, _p(A16), 0, None) == q4.Q4_OK
    assert lib.q4_pack(_p(A16), 0, 64, _p(A16), _p(A16), _p(A16), None) == q4.Q4_OK
    assert lib.q4_multilinear_step(_p(A16), 2, _p(A16), _p(A16), _p(A16), 16, 0, 64, 3, _p(A16), 1, None) == q4.Q4_OK


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        q4.q4_pack(w)


def _chain(n_stages=2, k=256, n=16, x=A16, y=Y16, packed=A16):
    stages = (q4._ChainStage * n_stages)(*[q4._ChainStage(x, k, i, 1) for i in range(n_stages)])
    mats = (q4._ChainMatrix * n_stages)(*[q4._ChainMatrix(packed, A16, A16, y, n) for _ in range(n_stages)])
    return stages, mats


def _stage_field(buf, s, off):
    base = 64 + 64 * s
    return int.from_bytes(bytes(buf[base + off:base + off + 4]), "little", signed=True)


def test_chain_encode_validation_and_layout():
    lib = q4.load()
    assert lib.q4_chain_plan_bytes(0, 1) < 0
    nb = lib.q4_chain_plan_bytes(2, 2)
    assert nb == 64 + 2 * 64 + 2 * 48
    buf = (ctypes.c_uint8 * nb)()
    stages, mats = _chain()
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    hdr = bytes(buf[:16])
    assert int.from_bytes(hdr[0:4], "little") == 0x34433451
    assert int.from_bytes(hdr[4:8], "little") == 2
    # too small a buffer, bad dtype, misaligned x, k not a multiple of 32, stage coverage errors
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 0, ctypes.byref(buf), nb - 1) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_encode(ctypes.byref(stages), 2, ctypes.byref(mats), 2, 5, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s2, m2 = _chain(x=ODD)
    assert lib.q4_chain_encode(ctypes.byref(s2), 2, ctypes.byref(m2), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_ALIGN
    s3, m3 = _chain(k=40)
    assert lib.q4_chain_encode(ctypes.byref(s3), 2, ctypes.byref(m3), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s4, m4 = _chain()
    s4[1].first_matrix = 0
    assert lib.q4_chain_encode(ctypes.byref(s4), 2, ctypes.byref(m4), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_SHAPE
    s6, m6 = _chain(k=96)  # 3 groups: one chunk, mostly past the row end
    assert lib.q4_chain_encode(ctypes.byref(s6), 2, ctypes.byref(m6), 2, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    # the LDS copy of the plan bounds stages and matrices
    big = lib.q4_chain_plan_bytes(385, 385)
    bigbuf = (ctypes.c_uint8 * big)()
    s9, m9 = _chain(n_stages=385)
    assert lib.q4_chain_encode(ctypes.byref(s9), 385, ctypes.byref(m9), 385, 0, ctypes.byref(bigbuf), big) == q4.Q4_ERR_UNSUPPORTED
    ok = lib.q4_chain_plan_bytes(384, 384)
    okbuf = (ctypes.c_uint8 * ok)()
    s10, m10 = _chain(n_stages=384)
    assert lib.q4_chain_encode(ctypes.byref(s10), 384, ctypes.byref(m10), 384, 0, ctypes.byref(okbuf), ok) == q4.Q4_OK
    s5, m5 = _chain(packed=0)
    assert lib.q4_chain_encode(ctypes.byref(s5), 2, ctypes.byref(m5), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_NULL
    s7, m7 = _chain(y=A16)  # a stage writing its own input
    assert lib.q4_chain_encode(ctypes.byref(s7), 2, ctypes.byref(m7), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_UNSUPPORTED
    s8, m8 = _chain(k=12288 + 256, n=64)  # wider than the executor's activation buffer
    assert lib.q4_chain_encode(ctypes.byref(s8), 2, ctypes.byref(m8), 2, 0, ctypes.byref(buf), nb) == q4.Q4_ERR_UNSUPPORTED


def test_chain_encode_rows_validation():
    """Several activation rows: the row count is checked and stored in the
    plan's header (int32 at byte 20), the executor's lower limits for 2..4
    rows are enforced, and buffer overlap is judged on m_rows rows."""
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(2, 2)
    buf = (ctypes.c_uint8 * nb)()

    def enc(stages, mats, m, ns=2, b=buf, size=nb):
        return lib.q4_chain_encode_rows(ctypes.byref(stages), ns, ctypes.byref(mats), ns, m, 0, ctypes.byref(b), size)

    stages, mats = _chain()
    for m in (0, 5, -1):
        assert enc(stages, mats, m) == q4.Q4_ERR_SHAPE
    for m in (1, 2, 3, 4):
        assert enc(stages, mats, m) == q4.Q4_OK
        assert int.from_bytes(bytes(buf[20:24]), "little") == m
    s1, m1 = _chain(k=11264, n=64)
    assert enc(s1, m1, 4) == q4.Q4_OK
    s2, m2 = _chain(k=11264 + 32, n=64)  # wider than the multi-row activation buffer
    assert enc(s2, m2, 2) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s2, m2, 1) == q4.Q4_OK
    # y starts one bf16 row of x past x: disjoint for one row, overlapping for two
    s3, m3 = _chain(k=256, n=16, y=A16 + 2 * 256)
    assert enc(s3, m3, 1) == q4.Q4_OK
    assert enc(s3, m3, 2) == q4.Q4_ERR_UNSUPPORTED
    # the LDS plan tables hold 128 stages for several rows (384 for one)
    n129 = lib.q4_chain_plan_bytes(129, 129)
    b129 = (ctypes.c_uint8 * n129)()
    s4, m4 = _chain(n_stages=129)
    assert enc(s4, m4, 2, 129, b129, n129) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s4, m4, 1, 129, b129, n129) == q4.Q4_OK
    n128 = lib.q4_chain_plan_bytes(128, 128)
    b128 = (ctypes.c_uint8 * n128)()
    s5, m5 = _chain(n_stages=128)
    assert enc(s5, m5, 4, 128, b128, n128) == q4.Q4_OK
    # 32 units of 4 rows per block: n up to 32 * 4 * 256 compute units
    s6, m6 = _chain(n=32 * 4 * 256)
    assert enc(s6, m6, 2) == q4.Q4_OK
    s7, m7 = _chain(n=32 * 4 * 256 + 4)
    assert enc(s7, m7, 2) == q4.Q4_ERR_UNSUPPORTED
    assert enc(s7, m7, 1) == q4.Q4_OK


def test_chain_run_rows_validation():
    lib = q4.load()
    for m in (0, 5):
        assert lib.q4_chain_run_rows(_p(A16), m, 0, _p(A16), None) == q4.Q4_ERR_SHAPE
    assert lib.q4_chain_run_rows(None, 2, 0, _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_chain_run_rows(_p(A16), 2, 3, _p(A16), None) == q4.Q4_ERR_SHAPE


def test_chain_stage_geometry_and_dependencies():
    """Lanes per row and chunk count per stage, and the dependency flags the
    encoder derives from buffer overlap: stage 1 reads stage 0's output."""
    lib = q4.load()
    nb = lib.q4_chain_plan_bytes(3, 3)
    buf = (ctypes.c_uint8 * nb)()
    Y0, Y1, Y2 = 0x400000, 0x800000, 0xC00000
    stages = (q4._ChainStage * 3)(q4._ChainStage(A16, 4096, 0, 1), q4._ChainStage(Y0, 11264, 1, 1),
                                   q4._ChainStage(A16 + 0x100000, 2816, 2, 1))
    mats = (q4._ChainMatrix * 3)(q4._ChainMatrix(A16, A16, A16, Y0, 11264), q4._ChainMatrix(A16, A16, A16, Y1, 4096),
                                 q4._ChainMatrix(A16, A16, A16, Y2, 1024))
    assert lib.q4_chain_encode(ctypes.byref(stages), 3, ctypes.byref(mats), 3, 0, ctypes.byref(buf), nb) == q4.Q4_OK
    # G, c_log2, CH at byte offsets 8, 12, 16; x_internal 28, sync_outputs 32
    # (16 lanes per row, chunks of 16 groups: CH = ceil(G / 16))
    assert [_stage_field(buf, 0, o) for o in (8, 12, 16)] == [128, 4, 8]
    assert [_stage_field(buf, 1, o) for o in (8, 12, 16)] == [352, 4, 22]
    assert [_stage_field(buf, 2, o) for o in (8, 12, 16)] == [88, 4, 6]     # ragged last chunk
    assert [_stage_field(buf, s, 28) for s in range(3)] == [0, 1, 0]
    assert [_stage_field(buf, s, 32) for s in range(3)] == [1, 0, 0]


def test_chain_run_validation():
    lib = q4.load()
    assert lib.q4_chain_run(None, 0, _p(A16), None) == q4.Q4_ERR_NULL
    assert lib.q4_chain_run(_p(A16), 0, _p(A16 + 64), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_chain_run(_p(A16 + 16), 0, _p(A16), None) == q4.Q4_ERR_ALIGN
    assert lib.q4_chain_run(_p(A16), 3, _p(A16), None) == q4.Q4_ERR_SHAPE
